// Host runtime of the C ABI declared in include/uly.h: argument checks, the
// tagged target cache, the comm stream and the grouped completion
// handshake, launch bookkeeping and per-kernel event timing.
//
// Pages cited (by title and section):
//  [CA]  TeleFuser documentation, "Communication Architecture" — "Ulysses"
//        (the maps and their divisibility checks, done before any
//        communication), "Stream ordering protocol" and "Efficiency
//        Invariants" (stream events instead of device-wide syncs, Q/K/V all
//        submitted before anyone waits).
//  [P27] TeleFuser PR #27, "Changes Made" (cached targets keyed by tag,
//        shape, dtype, mode and device, up to 12; one grouped handshake;
//        V submitted before Q/K norm and RoPE) and "Description".
//  [UC]  flashinfer UlyssesCommunicator(backend="pcie") PR, "Failure
//        envelope" (argument rejections decided before native work, fail-
//        stop after a transport failure) and "element type".

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "uly.h"
#include "uly_internal.h"
#include "uly_proj.h"

using namespace uly;

namespace {

thread_local std::string g_err;

uly_status fail(uly_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

constexpr int kMaxTargetsCap = 12;   // [P27 "Changes Made"]
constexpr int kTagMax = 63;
constexpr int64_t kMaxVecs = int64_t(1) << 31;   // per launch plan, keeps 32-bit indexing exact
constexpr int kMaxWorld = 4096;                  // emulated ranks per context
// Bound on any element count or byte size formed from caller extents (far
// beyond any device's memory).  Sizes below it leave room for the further
// products by P, the element size and 16 that the plans form, in int64.
constexpr int64_t kMaxExtent = int64_t(1) << 48;

// The product of non-negative factors, or -1 when a factor is negative or the
// product passes kMaxExtent.  Checked factor by factor, so no product wraps.
int64_t checked_prod(std::initializer_list<int64_t> f) {
    int64_t r = 1;
    for (int64_t v : f)
        if (v < 0 || __builtin_mul_overflow(r, v, &r) || r > kMaxExtent) return -1;
    return r;
}

struct Target {
    std::string tag;
    int mode;
    int dtype;
    int64_t shape[4];
    int device;
    void *ptr;
    size_t bytes;
};

struct Pending {
    hipStream_t stream;   // a stream that carries work of the current group
};

struct ProfRecord {
    int kind;
    hipEvent_t start;
    hipEvent_t stop;
    double ms;     // < 0 until measured
};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 16-bit floats, or opaque single bytes (fp8 / int8 payloads, [UC "element type"]).
bool valid_dtype(int dtype) { return dtype == ULY_F16 || dtype == ULY_BF16 || dtype == ULY_U8; }
int64_t elem_size(int dtype) { return dtype == ULY_U8 ? 1 : 2; }

struct Range {
    uintptr_t lo = 0, hi = 0;   // [lo, hi), empty when lo == hi
    bool overlaps(const Range &o) const { return lo < hi && o.lo < o.hi && lo < o.hi && o.lo < hi; }
};

// A checked rank-major 4-D operand.
struct Operand {
    const uint8_t *data = nullptr;
    int dtype = 0;
    int64_t rank_stride = 0;
    int64_t B = 0, S = 0, H = 0, D = 0;
    int64_t sb = 0, ss = 0, sh = 0;   // element strides
    int64_t es = 2;                   // bytes per element
    Range range;
    bool empty() const { return B == 0 || S == 0; }
};

uly_status check_operand(const uly_tensor *t, const char *name, int P, Operand &o) {
    if (!t) return fail(ULY_E_INVAL, "%s: null descriptor", name);
    if (!valid_dtype(t->dtype)) return fail(ULY_E_DTYPE, "%s: unknown dtype %d", name, t->dtype);
    if (t->reserved != 0) return fail(ULY_E_INVAL, "%s: reserved field must be 0", name);
    for (int i = 0; i < 4; ++i)
        if (t->shape[i] < 0) return fail(ULY_E_INVAL, "%s: negative extent in dim %d", name, i);
    if (t->shape[2] < 1 || t->shape[3] < 1)
        return fail(ULY_E_INVAL, "%s: H and D must be positive", name);
    if (t->stride[3] != 1) return fail(ULY_E_INVAL, "%s: head-dim stride must be 1", name);
    if (t->rank_stride < 0 || t->stride[0] < 0 || t->stride[1] < 0 || t->stride[2] < 0)
        return fail(ULY_E_INVAL, "%s: negative stride", name);
    const int64_t es = elem_size(t->dtype);
    // Bounded extents and strides keep every size and offset formed below in int64.
    if (checked_prod({P, t->shape[0], t->shape[1], t->shape[2], t->shape[3], es}) < 0 ||
        checked_prod({P, t->shape[1]}) < 0 || checked_prod({t->shape[2], t->shape[3], es}) < 0 ||
        t->shape[0] > kMaxExtent || t->rank_stride > kMaxExtent || t->stride[0] > kMaxExtent || t->stride[1] > kMaxExtent ||
        t->stride[2] > kMaxExtent)
        return fail(ULY_E_UNSUPPORTED, "%s: extents or strides too large", name);
    if ((t->shape[3] * es) % 16 != 0)
        return fail(ULY_E_INVAL, "%s: a head row of %lld bytes is not a multiple of 16", name,
                    (long long)(t->shape[3] * es));
    const int64_t ext[4] = {P, t->shape[0], t->shape[1], t->shape[2]};
    const int64_t str[4] = {t->rank_stride, t->stride[0], t->stride[1], t->stride[2]};
    for (int i = 0; i < 4; ++i)
        if (ext[i] > 1 && (str[i] * es) % 16 != 0)
            return fail(ULY_E_INVAL, "%s: byte stride of dim %d (%lld) is not a multiple of 16", name,
                        i, (long long)(str[i] * es));
    o.data = static_cast<const uint8_t *>(t->data);
    o.dtype = t->dtype;
    o.es = es;
    o.rank_stride = t->rank_stride;
    o.B = t->shape[0];
    o.S = t->shape[1];
    o.H = t->shape[2];
    o.D = t->shape[3];
    o.sb = t->stride[0];
    o.ss = t->stride[1];
    o.sh = t->stride[2];
    if (!o.empty()) {
        if (!o.data) return fail(ULY_E_INVAL, "%s: null data pointer", name);
        if (!aligned16(o.data)) return fail(ULY_E_INVAL, "%s: data pointer not 16-byte aligned", name);
        int64_t maxoff = o.D - 1;
        for (int i = 0; i < 4; ++i) {
            const int64_t span = checked_prod({ext[i] - 1, str[i], es});
            if (span < 0) return fail(ULY_E_UNSUPPORTED, "%s: strides too large", name);
            maxoff += span / es;      // at most 4 terms below 2^48: no wrap
        }
        o.range.lo = reinterpret_cast<uintptr_t>(o.data);
        o.range.hi = o.range.lo + uintptr_t(maxoff + 1) * uintptr_t(es);
    }
    return ULY_OK;
}

Range byte_range(const void *p, int64_t bytes) {
    Range r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + uintptr_t(bytes);
    return r;
}

struct DeviceGuard {
    int prev = -1;
    int dev;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int d) : dev(d) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
    }
};

}  // namespace

struct uly_ctx {
    int device = -1;
    int P = 1;
    int max_targets = kMaxTargetsCap;
    bool host_only = true;
    bool broken = false;
    hipStream_t comm = nullptr;
    hipEvent_t fork_ev = nullptr;
    std::vector<Target> targets;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> sync_pool;
    int profile_mask = 0;   // bit k: bracket kernels of kind k with timing events
    int profile_every = 1;  // time one launch in this many of each timed kind
    int64_t profile_seen[ULY_K_COUNT] = {};
    std::vector<ProfRecord> prof;
    std::vector<hipEvent_t> timing_pool;
    uly_stats stats{};
    int fail_after = -1;
    int route = ULY_ROUTE_KERNEL;   // how ulysses_scatter_qkv moves its operands
    int proj_ring = 0;              // token-row ring depth of the projection: 0 automatic, else 2 or 3
};

namespace {

uly_status ctx_ok(uly_ctx *c) {
    if (!c) return fail(ULY_E_INVAL, "null context");
    if (c->broken) return fail(ULY_E_BROKEN, "context is broken by an earlier failure; destroy it");
    return ULY_OK;
}

uly_status poison(uly_ctx *c, hipError_t e, const char *what) {
    c->broken = true;
    return fail(ULY_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_tag(const char *tag) { return tag && tag[0] && strlen(tag) <= size_t(kTagMax); }

Target *find_target(uly_ctx *c, const char *tag, int mode, int dtype, const int64_t shape[4]) {
    for (auto &t : c->targets)
        if (t.mode == mode && t.dtype == dtype && t.device == c->device && t.tag == tag &&
            t.shape[0] == shape[0] && t.shape[1] == shape[1] && t.shape[2] == shape[2] &&
            t.shape[3] == shape[3])
            return &t;
    return nullptr;
}

// Destination of one member: explicit pointer or the cached target of its key.
uly_status resolve_target(uly_ctx *c, const char *name, const char *tag, void *explicit_out,
                          int mode, int dtype, const int64_t shape[4], uint8_t *&out) {
    if (explicit_out) {
        if (!aligned16(explicit_out)) return fail(ULY_E_INVAL, "%s: destination not 16-byte aligned", name);
        out = static_cast<uint8_t *>(explicit_out);
        return ULY_OK;
    }
    if (!valid_tag(tag)) return fail(ULY_E_INVAL, "%s: no destination and no valid tag", name);
    c->stats.lookups++;
    Target *t = find_target(c, tag, mode, dtype, shape);
    if (!t) {
        // A tag registered with another dtype is a dtype error, not a miss ([UC] "element type").
        for (auto &o : c->targets)
            if (o.tag == tag && o.mode == mode && o.dtype != dtype && o.shape[0] == shape[0] &&
                o.shape[1] == shape[1] && o.shape[2] == shape[2] && o.shape[3] == shape[3])
                return fail(ULY_E_DTYPE, "%s: target '%s' is registered with dtype %d, call uses %d",
                            name, tag, o.dtype, dtype);
        return fail(ULY_E_NOT_FOUND,
                    "%s: no target registered for tag '%s' mode %d dtype %d shape [%lld,%lld,%lld,%lld]",
                    name, tag, mode, dtype, (long long)shape[0], (long long)shape[1],
                    (long long)shape[2], (long long)shape[3]);
    }
    c->stats.hits++;
    out = static_cast<uint8_t *>(t->ptr);
    return ULY_OK;
}

// Timing events only measure: they need no system-scope fence (an L2
// write-back and invalidate each time one is recorded, which would both
// lengthen the bracketed interval and slow the launches after it).
constexpr unsigned kTimingEventFlags = hipEventDisableSystemFence;

hipEvent_t take_event(std::vector<hipEvent_t> &pool, unsigned flags, hipError_t &err) {
    if (!pool.empty()) {
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    err = hipEventCreateWithFlags(&e, flags);
    return err == hipSuccess ? e : nullptr;
}

// Fault injection (uly_debug_fail_launch): true when this launch must fail.
bool injected_failure(uly_ctx *c) {
    if (c->fail_after == 0) {
        c->fail_after = -1;
        c->broken = true;
        fail(ULY_E_HIP, "injected launch failure (test hook)");
        return true;
    }
    if (c->fail_after > 0) --c->fail_after;
    return false;
}

// What a host-only context returns where a device context would launch.
uly_status host_only_launch(uly_ctx *c) {
    if (injected_failure(c)) return ULY_E_HIP;
    return fail(ULY_E_UNSUPPORTED, "host-only context cannot launch");
}

// Enqueue one kernel through `enqueue`, with optional timing events and the
// fail-stop bookkeeping.
template <class F>
uly_status launch(uly_ctx *c, int kind, hipStream_t s, F &&enqueue) {
    if (injected_failure(c)) return ULY_E_HIP;
    (void)hipGetLastError();   // clear a stale error left by someone else's call
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipSuccess;
    const bool timed = ((c->profile_mask >> kind) & 1) && (c->profile_seen[kind]++ % c->profile_every == 0);
    if (timed) {
        e0 = take_event(c->timing_pool, kTimingEventFlags, err);
        if (!e0) return poison(c, err, "hipEventCreate");
        e1 = take_event(c->timing_pool, kTimingEventFlags, err);
        if (!e1) return poison(c, err, "hipEventCreate");
        if ((err = hipEventRecord(e0, s)) != hipSuccess) return poison(c, err, "hipEventRecord");
    }
    enqueue();
    err = hipGetLastError();
    if (err != hipSuccess) return poison(c, err, "kernel launch");
    if (timed) {
        if ((err = hipEventRecord(e1, s)) != hipSuccess) return poison(c, err, "hipEventRecord");
        c->prof.push_back({kind, e0, e1, -1.0});
    }
    c->stats.launches++;
    return ULY_OK;
}

// Note that `s` carries work of the current group.  The event that the
// consumer waits on is recorded at uly_wait time, and only for streams other
// than the consumer's, so a group that runs entirely on the consumer's
// stream costs no event at all.
uly_status mark_pending(uly_ctx *c, hipStream_t s) {
    for (auto &p : c->pending)
        if (p.stream == s) return ULY_OK;
    c->pending.push_back({s});
    return ULY_OK;
}

// The comm stream waits for everything enqueued on `caller` so far (input
// readiness and the reuse hazard of the targets it is about to overwrite).
uly_status fork_comm(uly_ctx *c, hipStream_t caller) {
    hipError_t err = hipEventRecord(c->fork_ev, caller);
    if (err != hipSuccess) return poison(c, err, "hipEventRecord");
    err = hipStreamWaitEvent(c->comm, c->fork_ev, 0);
    return err == hipSuccess ? ULY_OK : poison(c, err, "hipStreamWaitEvent");
}

#ifndef ULY_SCATTER_ORDER
#define ULY_SCATTER_ORDER 0
#endif
#ifndef ULY_GATHER_ORDER
#define ULY_GATHER_ORDER 0
#endif

// Fill a plan from 4 (extent, source stride, destination stride) dims,
// outermost first; strides in bytes.
void fill_plan(CopyPlan &p, const uint8_t *src, uint8_t *dst, const int64_t n[4], const int64_t ss[4],
               const int64_t ds[4], int64_t vpc, int64_t total) {
    p = CopyPlan{};
    p.src = src;
    p.dst = dst;
    for (int k = 0; k < 4; ++k) {
        p.ss[k] = ss[k];
        p.ds[k] = ds[k];
    }
    p.vpc = FastDiv::make(uint32_t(vpc));
    p.n1 = FastDiv::make(uint32_t(n[1]));
    p.n2 = FastDiv::make(uint32_t(n[2]));
    p.n3 = FastDiv::make(uint32_t(n[3]));
    p.total = uint32_t(total);
}

// Plan of one scatter member: rank-major source [P(r)][B][S_l][H][D]
// (strided) -> dense [P(q)][B][P(r)*S_l][Hl][D].  A chunk is one token's
// head band q: Hl*D elements.
uly_status plan_scatter(const Operand &x, int P, uint8_t *dst, CopyPlan &p) {
    const int64_t Hl = x.H / P, S = int64_t(P) * x.S;
    const int64_t C = Hl * x.D * x.es;   // chunk bytes
    const int64_t total = int64_t(P) * x.B * P * x.S * (C / 16);
    if (total >= kMaxVecs || x.S >= kMaxVecs || x.B >= kMaxVecs)
        return fail(ULY_E_UNSUPPORTED, "operand too large for one launch (%lld vectors)", (long long)total);
    // per-dim (source, destination) byte strides
    const int64_t q_s = Hl * x.sh * x.es, q_d = x.B * S * C;
    const int64_t b_s = x.sb * x.es, b_d = S * C;
    const int64_t r_s = x.rank_stride * x.es, r_d = x.S * C;
    const int64_t s_s = x.ss * x.es, s_d = C;
    if (ULY_SCATTER_ORDER == 0) {     // destination order (q, b, r, s)
        const int64_t n[4] = {P, x.B, P, x.S}, ss[4] = {q_s, b_s, r_s, s_s}, ds[4] = {q_d, b_d, r_d, s_d};
        fill_plan(p, x.data, dst, n, ss, ds, C / 16, total);
    } else {                          // source order (r, b, s, q)
        const int64_t n[4] = {P, x.B, x.S, P}, ss[4] = {r_s, b_s, s_s, q_s}, ds[4] = {r_d, b_d, s_d, q_d};
        fill_plan(p, x.data, dst, n, ss, ds, C / 16, total);
    }
    return ULY_OK;
}

// Plan of the inverse: head-sharded [P(q)][B][S][Hl][D] (strided) -> dense
// [P(r)][B][S_l][P(q)*Hl][D].
uly_status plan_gather(const Operand &o, int P, uint8_t *dst, CopyPlan &p) {
    const int64_t S_l = o.S / P, H = o.H * P;
    const int64_t C = o.H * o.D * o.es;
    const int64_t total = int64_t(P) * o.B * S_l * P * (C / 16);
    if (total >= kMaxVecs || o.S >= kMaxVecs || o.B >= kMaxVecs)
        return fail(ULY_E_UNSUPPORTED, "operand too large for one launch (%lld vectors)", (long long)total);
    const int64_t r_s = S_l * o.ss * o.es, r_d = o.B * S_l * H * o.D * o.es;
    const int64_t b_s = o.sb * o.es, b_d = S_l * H * o.D * o.es;
    const int64_t s_s = o.ss * o.es, s_d = H * o.D * o.es;
    const int64_t q_s = o.rank_stride * o.es, q_d = C;
    if (ULY_GATHER_ORDER == 0) {      // destination order (r, b, s, q)
        const int64_t n[4] = {P, o.B, S_l, P}, ss[4] = {r_s, b_s, s_s, q_s}, ds[4] = {r_d, b_d, s_d, q_d};
        fill_plan(p, o.data, dst, n, ss, ds, C / 16, total);
    } else {                          // source order (q, b, r, s)
        const int64_t n[4] = {P, o.B, P, S_l}, ss[4] = {q_s, b_s, r_s, s_s}, ds[4] = {q_d, b_d, r_d, s_d};
        fill_plan(p, o.data, dst, n, ss, ds, C / 16, total);
    }
    return ULY_OK;
}

// Copy-engine form of one scatter member: block (r, q, b) is S_l rows of
// Hl*D elements at the source token pitch, landing as one dense run in the
// destination [P(q)][B][S][Hl][D].
hipError_t copy_engine_scatter(const Operand &x, int P, uint8_t *dst, hipStream_t s) {
    const int64_t Hl = x.H / P, S = int64_t(P) * x.S, C = Hl * x.D * x.es;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t q = 0; q < P; ++q)
            for (int64_t b = 0; b < x.B; ++b) {
                const uint8_t *src = x.data + x.es * (r * x.rank_stride + b * x.sb + q * Hl * x.sh);
                uint8_t *d = dst + ((q * x.B + b) * S + r * x.S) * C;
                const size_t pitch = x.S > 1 ? size_t(x.ss * x.es) : size_t(C);
                hipError_t e = hipMemcpy2DAsync(d, size_t(C), src, pitch, size_t(C), size_t(x.S),
                                                hipMemcpyDeviceToDeviceNoCU, s);
                if (e != hipSuccess) return e;
            }
    return hipSuccess;
}

uly_status finish_batch(CopyBatch &b) {
    uint64_t blocks = 0;
    for (int i = 0; i < b.n; ++i) {
        b.p[i].first_block = uint32_t(blocks);
        blocks += (b.p[i].total + kCopyVecsPerBlock - 1) / kCopyVecsPerBlock;
    }
    if (blocks >= (uint64_t(1) << 31)) return fail(ULY_E_UNSUPPORTED, "grid too large");
    b.blocks = uint32_t(blocks);
    return ULY_OK;
}

uly_status check_overlaps(const std::vector<Range> &in, const std::vector<Range> &out) {
    for (size_t i = 0; i < out.size(); ++i) {
        for (const Range &r : in)
            if (out[i].overlaps(r)) return fail(ULY_E_OVERLAP, "an input overlaps destination %zu", i);
        for (size_t j = i + 1; j < out.size(); ++j)
            if (out[i].overlaps(out[j])) return fail(ULY_E_OVERLAP, "destinations %zu and %zu overlap", i, j);
    }
    return ULY_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char *uly_last_error(void) { return g_err.c_str(); }

const char *uly_status_string(int st) {
    switch (st) {
    case ULY_OK: return "ULY_OK";
    case ULY_E_INVAL: return "ULY_E_INVAL";
    case ULY_E_DTYPE: return "ULY_E_DTYPE";
    case ULY_E_CACHE_FULL: return "ULY_E_CACHE_FULL";
    case ULY_E_NOT_FOUND: return "ULY_E_NOT_FOUND";
    case ULY_E_UNSUPPORTED: return "ULY_E_UNSUPPORTED";
    case ULY_E_HIP: return "ULY_E_HIP";
    case ULY_E_BROKEN: return "ULY_E_BROKEN";
    case ULY_E_OVERLAP: return "ULY_E_OVERLAP";
    default: return "unknown status";
    }
}

uly_status uly_create(uly_ctx **out, int device, int world_size, int max_targets) {
    if (!out) return fail(ULY_E_INVAL, "null output pointer");
    *out = nullptr;
    if (world_size < 1 || world_size > kMaxWorld)
        return fail(ULY_E_INVAL, "world_size must be in [1, %d] (got %d)", kMaxWorld, world_size);
    if (max_targets < 1 || max_targets > kMaxTargetsCap)
        return fail(ULY_E_INVAL, "max_targets must be in [1, %d] (got %d)", kMaxTargetsCap, max_targets);
    if (device < -1) return fail(ULY_E_INVAL, "device must be >= -1 (got %d)", device);
    uly_ctx *c = new uly_ctx();
    c->device = device;
    c->P = world_size;
    c->max_targets = max_targets;
    c->host_only = device < 0;
    if (!c->host_only) {
        int n = 0;
        hipError_t err = hipGetDeviceCount(&n);
        if (err != hipSuccess || device >= n) {
            delete c;
            return err != hipSuccess ? fail(ULY_E_HIP, "hipGetDeviceCount: %s", hipGetErrorString(err))
                                     : fail(ULY_E_INVAL, "device %d out of range (%d devices)", device, n);
        }
        DeviceGuard g(device);
        if (g.err != hipSuccess) {
            delete c;
            return fail(ULY_E_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
        }
        // Default priority on purpose: the overlap comes from two streams,
        // not from a priority difference.
        err = hipStreamCreateWithFlags(&c->comm, hipStreamNonBlocking);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming);
        if (err != hipSuccess) {
            if (c->comm) (void)hipStreamDestroy(c->comm);
            delete c;
            return fail(ULY_E_HIP, "stream/event creation: %s", hipGetErrorString(err));
        }
    }
    *out = c;
    return ULY_OK;
}

uly_status uly_destroy(uly_ctx *c) {
    if (!c) return ULY_OK;
    uly_status st = ULY_OK;
    if (!c->host_only) {
        DeviceGuard g(c->device);
        if (c->comm && hipStreamSynchronize(c->comm) != hipSuccess)
            st = fail(ULY_E_HIP, "hipStreamSynchronize on destroy failed");
        for (auto e : c->sync_pool) (void)hipEventDestroy(e);
        for (auto &r : c->prof) {
            (void)hipEventDestroy(r.start);
            (void)hipEventDestroy(r.stop);
        }
        for (auto e : c->timing_pool) (void)hipEventDestroy(e);
        if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
        if (c->comm) (void)hipStreamDestroy(c->comm);
    }
    delete c;
    return st;
}

uly_status uly_target_register(uly_ctx *c, const char *tag, int mode, int dtype, const int64_t shape[4],
                               void *storage, size_t bytes) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (!valid_tag(tag)) return fail(ULY_E_INVAL, "tag must be 1..%d bytes", kTagMax);
    if (mode != ULY_MODE_SCATTER && mode != ULY_MODE_GATHER) return fail(ULY_E_INVAL, "bad mode %d", mode);
    if (!valid_dtype(dtype)) return fail(ULY_E_DTYPE, "bad dtype %d", dtype);
    if (!shape) return fail(ULY_E_INVAL, "null shape");
    int64_t elems = c->P;
    for (int i = 0; i < 4; ++i) {
        if (shape[i] < 1) return fail(ULY_E_INVAL, "target extents must be positive");
        if (elems > (int64_t(1) << 56) / shape[i]) return fail(ULY_E_INVAL, "target extents overflow");
        elems *= shape[i];
    }
    if (!storage || !aligned16(storage)) return fail(ULY_E_INVAL, "storage null or not 16-byte aligned");
    if (bytes < size_t(elems * elem_size(dtype)))
        return fail(ULY_E_INVAL, "storage of %zu bytes is smaller than the %lld bytes of P slabs", bytes,
                    (long long)(elems * elem_size(dtype)));
    if (find_target(c, tag, mode, dtype, shape))
        return fail(ULY_E_INVAL, "target '%s' with this key is already registered", tag);
    if (int(c->targets.size()) >= c->max_targets)
        return fail(ULY_E_CACHE_FULL, "target cache holds its maximum of %d entries", c->max_targets);
    Target t;
    t.tag = tag;
    t.mode = mode;
    t.dtype = dtype;
    for (int i = 0; i < 4; ++i) t.shape[i] = shape[i];
    t.device = c->device;
    t.ptr = storage;
    t.bytes = bytes;
    c->targets.push_back(t);
    c->stats.registrations++;
    return ULY_OK;
}

uly_status uly_target_lookup(uly_ctx *c, const char *tag, int mode, int dtype, const int64_t shape[4],
                             void **storage) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (!storage || !shape || !valid_tag(tag)) return fail(ULY_E_INVAL, "bad lookup arguments");
    *storage = nullptr;
    c->stats.lookups++;
    Target *t = find_target(c, tag, mode, dtype, shape);
    if (!t) return fail(ULY_E_NOT_FOUND, "no target for tag '%s'", tag);
    c->stats.hits++;
    *storage = t->ptr;
    return ULY_OK;
}

uly_status uly_target_count(uly_ctx *c, int *count) {
    if (!c || !count) return fail(ULY_E_INVAL, "null argument");
    *count = int(c->targets.size());
    return ULY_OK;
}

uly_status ulysses_scatter_qkv(uly_ctx *c, const uly_tensor *q, const uly_tensor *k, const uly_tensor *v,
                               const char *const tags[3], void *const outs[3], hipStream_t caller) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    const uly_tensor *mem[3] = {q, k, v};
    const char *names[3] = {"q", "k", "v"};
    Operand ops[3];
    uint8_t *dsts[3] = {nullptr, nullptr, nullptr};
    int present = 0, dtype = 0;
    int64_t B = -1, S = -1, D = -1;
    std::vector<Range> in_ranges, out_ranges;
    CopyBatch batch{};
    // Every member is checked and resolved before anything is enqueued.
    for (int i = 0; i < 3; ++i) {
        if (!mem[i]) continue;
        if ((st = check_operand(mem[i], names[i], c->P, ops[i])) != ULY_OK) return st;
        const Operand &x = ops[i];
        if (x.H % c->P != 0)
            return fail(ULY_E_INVAL, "%s: heads %lld not divisible by world size %d", names[i],
                        (long long)x.H, c->P);
        const int64_t Hl = x.H / c->P;
        if (Hl > 1 && x.sh != x.D)
            return fail(ULY_E_INVAL, "%s: heads of a token must be packed (stride[2] == D)", names[i]);
        if (present == 0) {
            dtype = x.dtype; B = x.B; S = x.S; D = x.D;
        } else {
            if (x.dtype != dtype) return fail(ULY_E_DTYPE, "%s: dtype differs from the other members", names[i]);
            if (x.B != B || x.S != S || x.D != D)
                return fail(ULY_E_INVAL, "%s: B, S_l and D must match the other members", names[i]);
        }
        ++present;
        const int64_t tshape[4] = {x.B, x.S * c->P, Hl, x.D};
        uint8_t *dst = nullptr;
        if (x.empty()) continue;
        if ((st = resolve_target(c, names[i], tags ? tags[i] : nullptr, outs ? outs[i] : nullptr,
                                 ULY_MODE_SCATTER, x.dtype, tshape, dst)) != ULY_OK)
            return st;
        dsts[i] = dst;
        in_ranges.push_back(x.range);
        out_ranges.push_back(byte_range(dst, int64_t(c->P) * tshape[0] * tshape[1] * tshape[2] * tshape[3] * x.es));
        if ((st = plan_scatter(x, c->P, dst, batch.p[batch.n])) != ULY_OK) return st;
        batch.n++;
    }
    if (present == 0) return fail(ULY_E_INVAL, "no operand given");
    if ((st = check_overlaps(in_ranges, out_ranges)) != ULY_OK) return st;
    if ((st = finish_batch(batch)) != ULY_OK) return st;
    if (c->host_only) return host_only_launch(c);
    if (batch.n == 0) return ULY_OK;
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    if (c->route == ULY_ROUTE_COPY_ENGINE)
        for (int i = 0; i < 3; ++i)
            if (mem[i] && !ops[i].empty() && ops[i].S > 1 && ops[i].ss < (ops[i].H / c->P) * ops[i].D)
                return fail(ULY_E_UNSUPPORTED, "%s: copy engines need a token pitch of at least one head band",
                            names[i]);
    if (c->route == ULY_ROUTE_CALLER) {
        // stream order on `caller` covers input readiness and target reuse
        if ((st = launch(c, ULY_K_SCATTER, caller, [&] { launch_relayout(batch, caller); })) != ULY_OK)
            return st;
        return mark_pending(c, caller);
    }
    if ((st = fork_comm(c, caller)) != ULY_OK) return st;
    if (c->route == ULY_ROUTE_COPY_ENGINE) {
        // One 2-D copy per (source rank, destination rank, batch) block, straight
        // into the final layout, on the copy engines instead of the compute units.
        hipError_t cerr = hipSuccess;
        st = launch(c, ULY_K_SCATTER, c->comm, [&] {
            for (int i = 0; i < 3 && cerr == hipSuccess; ++i) {
                if (!mem[i] || ops[i].empty()) continue;
                cerr = copy_engine_scatter(ops[i], c->P, dsts[i], c->comm);
            }
        });
        if (st != ULY_OK) return st;
        if (cerr != hipSuccess) return poison(c, cerr, "hipMemcpy2DAsync");
        return mark_pending(c, c->comm);
    }
    if ((st = launch(c, ULY_K_SCATTER, c->comm, [&] { launch_relayout(batch, c->comm); })) != ULY_OK)
        return st;
    return mark_pending(c, c->comm);
}

// The fused Q/K norm + RoPE scatter, into three targets or (packed) into one
// [P][B][S][Hl][3D] target whose head rows hold q, k and v side by side.
static uly_status fused_scatter(uly_ctx *c, const uly_tensor *q, const uly_tensor *k, const uly_tensor *v,
                                const void *w_q, const void *w_k, float eps, const float *cos_tab,
                                const float *sin_tab, int64_t table_rows, const char *const tags[3],
                                void *const outs[3], hipStream_t caller, bool packed) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    const uly_tensor *mem[3] = {q, k, v};
    const void *wts[3] = {w_q, w_k, nullptr};
    const char *names[3] = {"q", "k", "v"};
    Operand ops[3];
    uint8_t *dsts[3] = {nullptr, nullptr, nullptr};
    int present = 0, dtype = 0;
    int64_t B = -1, S = -1, D = -1;
    std::vector<Range> in_ranges, out_ranges;
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(ULY_E_INVAL, "eps must be a positive finite value");
    // Every member is checked and resolved before anything is enqueued.
    for (int i = 0; i < 3; ++i) {
        if (!mem[i]) continue;
        if ((st = check_operand(mem[i], names[i], c->P, ops[i])) != ULY_OK) return st;
        const Operand &x = ops[i];
        if (x.H % c->P != 0)
            return fail(ULY_E_INVAL, "%s: heads %lld not divisible by world size %d", names[i],
                        (long long)x.H, c->P);
        if (present == 0) {
            dtype = x.dtype; B = x.B; S = x.S; D = x.D;
        } else {
            if (x.dtype != dtype) return fail(ULY_E_DTYPE, "%s: dtype differs from the other members", names[i]);
            if (x.B != B || x.S != S || x.D != D)
                return fail(ULY_E_INVAL, "%s: B, S_l and D must match the other members", names[i]);
        }
        ++present;
        if (i < 2 && (!wts[i] || !aligned16(wts[i])))
            return fail(ULY_E_INVAL, "%s: weight pointer null or not 16-byte aligned", names[i]);
    }
    if (present == 0) return fail(ULY_E_INVAL, "no operand given");
    if (dtype == ULY_U8) return fail(ULY_E_UNSUPPORTED, "the fused norm + RoPE takes 16-bit operands");
    if (packed && (!q || !k || !v || ops[0].H != ops[1].H || ops[0].H != ops[2].H))
        return fail(ULY_E_INVAL, "the packed layout needs q, k and v with the same head count");
    const int lanes = int(D * 2 / 16);
    if (D % 2 != 0 || !(lanes == 4 || lanes == 8 || lanes == 16 || lanes == 32))
        return fail(ULY_E_UNSUPPORTED, "head dim %lld not supported (32, 64, 128 or 256)", (long long)D);
    if (!cos_tab || !sin_tab || !aligned16(cos_tab) || !aligned16(sin_tab))
        return fail(ULY_E_INVAL, "cos/sin tables null or not 16-byte aligned");
    if (table_rows < int64_t(c->P) * S)
        return fail(ULY_E_INVAL, "table has %lld rows, positions reach %lld", (long long)table_rows,
                    (long long)(int64_t(c->P) * S));
    if (checked_prod({table_rows, D / 2, 4}) < 0) return fail(ULY_E_UNSUPPORTED, "table too large");
    for (int i = 0; i < 3; ++i) {
        if (!mem[i] || ops[i].empty()) continue;
        const Operand &x = ops[i];
        in_ranges.push_back(x.range);
        if (packed && i > 0) {
            dsts[i] = dsts[0] + i * x.D * 2;     // the k and v columns of the one packed target
            continue;
        }
        const int64_t tshape[4] = {x.B, x.S * c->P, x.H / c->P, packed ? 3 * x.D : x.D};
        if ((st = resolve_target(c, packed ? "qkv" : names[i], tags ? tags[i] : nullptr,
                                 outs ? outs[i] : nullptr, ULY_MODE_SCATTER, x.dtype, tshape, dsts[i])) != ULY_OK)
            return st;
        out_ranges.push_back(byte_range(dsts[i], int64_t(c->P) * tshape[0] * tshape[1] * tshape[2] * tshape[3] * 2));
    }
    in_ranges.push_back(byte_range(cos_tab, table_rows * (D / 2) * 4));   // fp32 [rows][D/2]
    in_ranges.push_back(byte_range(sin_tab, table_rows * (D / 2) * 4));
    if (w_q) in_ranges.push_back(byte_range(w_q, D * 2));
    if (w_k) in_ranges.push_back(byte_range(w_k, D * 2));
    if ((st = check_overlaps(in_ranges, out_ranges)) != ULY_OK) return st;

    const int64_t Hall = (q ? ops[0].H : 0) + (k ? ops[1].H : 0) + (v ? ops[2].H : 0);
    const int64_t tokens = int64_t(c->P) * B * S;
    if (tokens >= kMaxVecs || checked_prod({tokens, Hall}) < 0 || tokens * Hall >= kMaxVecs)
        return fail(ULY_E_UNSUPPORTED, "too many rows for one launch (%lld tokens x %lld heads)", (long long)tokens,
                    (long long)Hall);

    NormRopeArgs a{};
    uint32_t Hrows[3] = {0, 0, 0};
    for (int i = 0; i < 3; ++i) {
        NormRopeOperand &o = a.op[i];
        o = NormRopeOperand{};
        o.hl = FastDiv::make(1);
        if (!mem[i] || ops[i].empty()) continue;
        const Operand &x = ops[i];
        const int64_t Hl = x.H / c->P, Sg = x.S * c->P;
        o.src = reinterpret_cast<const uint16_t *>(x.data);
        o.dst = reinterpret_cast<uint16_t *>(dsts[i]);
        // V rows are copied, but the kernel reads a weight row for every slot
        // without a branch: point V's at the table, which holds at least 2*D
        // readable bytes.
        o.w = static_cast<const uint16_t *>(wts[i] ? wts[i] : static_cast<const void *>(cos_tab));
        o.s_rank = x.rank_stride;
        o.s_b = x.sb;
        o.s_s = x.ss;
        o.s_h = x.sh;
        const int64_t row = packed ? 3 * x.D : x.D;    // destination elements per head row
        o.d_q = x.B * Sg * Hl * row;
        o.d_b = Sg * Hl * row;
        o.d_g = Hl * row;
        o.d_j = row;
        o.hl = FastDiv::make(uint32_t(Hl));
        o.H = uint32_t(x.H);
        Hrows[i] = uint32_t(x.H);
    }
    const uint32_t Hsum = Hrows[0] + Hrows[1] + Hrows[2];
    if (c->host_only) return host_only_launch(c);
    if (tokens == 0) return ULY_OK;
    a.cos_tab = cos_tab;
    a.sin_tab = sin_tab;
    a.rpt = FastDiv::make(Hsum);
    a.sl = FastDiv::make(uint32_t(S));
    a.bdiv = FastDiv::make(uint32_t(B));
    a.H0 = Hrows[0];
    a.H01 = Hrows[0] + Hrows[1];
    a.tokens = uint32_t(tokens);
    a.S_l = uint32_t(S);
    a.D = uint32_t(D);
    a.eps = eps;
    a.inv_D = 1.0f / float(D);
    const uint32_t blocks = uint32_t((tokens + kRopeTokens - 1) / kRopeTokens);
    // A wave holds 64 / lanes consecutive row slots; when every operand's
    // head count is a multiple of that, no wave straddles two operands.
    const uint32_t per_wave = uint32_t(64 / lanes);
    const bool uniform = Hrows[0] % per_wave == 0 && Hrows[1] % per_wave == 0 && Hrows[2] % per_wave == 0;
    // Tiles that never cross a rank or batch boundary need one decode per block.
    const bool tile = S % kRopeTokens == 0;
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    // Operands that are each one dense [P][B][S_l][H][D] tensor take the
    // operand-major band form (the blocks in flight then read one tensor front
    // to back); interleaved ones, such as Q/K/V views of a fused projection,
    // the token-tile form, which reads each token's rows of all operands at once.
    a.P = uint32_t(c->P);
    bool dense = true;
    for (int i = 0; i < 3; ++i) {
        if (!Hrows[i]) continue;
        const Operand &x = ops[i];
        dense = dense && x.sh == x.D && x.ss == x.H * x.D && x.sb == x.S * x.ss && x.rank_stride == x.B * x.sb;
    }
    const bool band = dense && lanes == 16 && S % kBandTokens == 0;
    // In the band form V, which is only copied, goes through the relayout
    // kernel right after, on the same stream: on dense operands it moves its
    // bytes at the plain copy rate, faster than as band blocks (the Wan-style
    // step: 995 us against 1030 us).  In the token-tile form V rides in the
    // same launch, which reads each token's rows of all operands together.
    // (A V of 2^31 vectors or more, beyond one relayout plan, stays in the band launch.)
    const int64_t v_vecs = Hrows[2] ? tokens * ops[2].H * ops[2].D * ops[2].es / 16 : 0;
    const bool v_apart = band && !packed && Hrows[2] != 0 && v_vecs < kMaxVecs;
    CopyBatch vbatch{};
    if (v_apart) {
        if ((st = plan_scatter(ops[2], c->P, dsts[2], vbatch.p[0])) != ULY_OK) return st;
        vbatch.n = 1;
        if ((st = finish_batch(vbatch)) != ULY_OK) return st;
    }
    uint32_t nops = 0;
    for (int i = 0; i < 3; ++i)
        if (Hrows[i] && !(v_apart && i == 2)) a.task_op[nops++] = uint32_t(i);
    for (uint32_t i = nops; i < 3; ++i) a.task_op[i] = nops ? a.task_op[0] : 0u;
    const uint32_t band_blocks = uint32_t(tokens / kBandTokens) * nops;
    if (nops > 0 &&
        (st = launch(c, ULY_K_NORM_ROPE, caller, [&] {
             if (band) launch_norm_rope_band(a, dtype, band_blocks, caller);
             else launch_norm_rope(a, lanes, dtype, uniform, tile, blocks, caller);
         })) != ULY_OK)
        return st;
    if (v_apart && (st = launch(c, ULY_K_SCATTER, caller, [&] { launch_relayout(vbatch, caller); })) != ULY_OK)
        return st;
    return mark_pending(c, caller);
}

uly_status fused_qk_norm_rope_scatter(uly_ctx *c, const uly_tensor *q, const uly_tensor *k, const uly_tensor *v,
                                      const void *w_q, const void *w_k, float eps, const float *cos_tab,
                                      const float *sin_tab, int64_t table_rows, const char *const tags[3],
                                      void *const outs[3], hipStream_t caller) {
    return fused_scatter(c, q, k, v, w_q, w_k, eps, cos_tab, sin_tab, table_rows, tags, outs, caller, false);
}

uly_status fused_qkv_norm_rope_scatter_packed(uly_ctx *c, const uly_tensor *q, const uly_tensor *k,
                                              const uly_tensor *v, const void *w_q, const void *w_k, float eps,
                                              const float *cos_tab, const float *sin_tab, int64_t table_rows,
                                              const char *tag, void *out, hipStream_t caller) {
    const char *tags[3] = {tag, nullptr, nullptr};
    void *outs[3] = {out, nullptr, nullptr};
    return fused_scatter(c, q, k, v, w_q, w_k, eps, cos_tab, sin_tab, table_rows, tags, outs, caller, true);
}

uly_status fused_qkv_proj_norm_rope_scatter(uly_ctx *c, const void *x, int dtype, int64_t B, int64_t S_l,
                                           int64_t hidden, const void *w_qkv, int64_t Hq, int64_t Hkv, int64_t D,
                                           const void *w_q, const void *w_k, float eps, const float *cos_tab,
                                           const float *sin_tab, int64_t table_rows, const char *const tags[3],
                                           void *const outs[3], hipStream_t caller) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (dtype != ULY_F16 && dtype != ULY_BF16) return fail(ULY_E_DTYPE, "the projection takes 16-bit floats");
    if (B < 0 || S_l < 0) return fail(ULY_E_INVAL, "negative B or S_l");
    if (Hq < 1 || Hkv < 1) return fail(ULY_E_INVAL, "q and k/v need at least one head each");
    if (checked_prod({c->P, B, S_l}) < 0 || checked_prod({c->P, S_l}) < 0 || Hq > kMaxExtent ||
        Hkv > kMaxExtent || hidden > kMaxExtent || table_rows > kMaxExtent)
        return fail(ULY_E_UNSUPPORTED, "too large for one launch");
    if (Hq % c->P != 0 || Hkv % c->P != 0)
        return fail(ULY_E_INVAL, "heads (%lld, %lld) not divisible by world size %d", (long long)Hq,
                    (long long)Hkv, c->P);
    if (D != kProjD) return fail(ULY_E_UNSUPPORTED, "the projection kernel is built for head dim %d", kProjD);
    if (hidden < kProjTileK || hidden % kProjTileK != 0)
        return fail(ULY_E_INVAL, "hidden %lld is not a positive multiple of %d", (long long)hidden, kProjTileK);
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(ULY_E_INVAL, "eps must be a positive finite value");
    const void *ptrs[4] = {x, w_qkv, w_q, w_k};
    const char *pnames[4] = {"x", "w_qkv", "w_q", "w_k"};
    for (int i = 0; i < 4; ++i)
        if (!ptrs[i] || !aligned16(ptrs[i]))
            return fail(ULY_E_INVAL, "%s: pointer null or not 16-byte aligned", pnames[i]);
    if (!cos_tab || !sin_tab || !aligned16(cos_tab) || !aligned16(sin_tab))
        return fail(ULY_E_INVAL, "cos/sin tables null or not 16-byte aligned");
    if (table_rows < int64_t(c->P) * S_l)
        return fail(ULY_E_INVAL, "table has %lld rows, positions reach %lld", (long long)table_rows,
                    (long long)(int64_t(c->P) * S_l));
    const int64_t M = int64_t(c->P) * B * S_l, N = (Hq + 2 * Hkv) * D;
    const int64_t tiles = (M + kProjTileT - 1) / kProjTileT, NH = Hq + 2 * Hkv;
    const int64_t NHB = (NH + kProjHeads - 1) / kProjHeads;
    const int64_t MK = checked_prod({M, hidden}), NK = checked_prod({N, hidden}), TB = checked_prod({tiles, NHB});
    constexpr int64_t k2G = int64_t(1) << 31;
    if (M >= k2G || hidden >= k2G || MK < 0 || NK < 0 || TB < 0 || TB >= k2G || MK / 8 >= k2G || NK / 8 >= k2G)
        return fail(ULY_E_UNSUPPORTED, "too large for one launch");
    const char *names[3] = {"q", "k", "v"};
    const int64_t heads[3] = {Hq, Hkv, Hkv};
    uint8_t *dsts[3] = {nullptr, nullptr, nullptr};
    std::vector<Range> in_ranges{byte_range(x, M * hidden * 2), byte_range(w_qkv, N * hidden * 2),
                                 byte_range(w_q, D * 2), byte_range(w_k, D * 2),
                                 byte_range(cos_tab, table_rows * (D / 2) * 4),
                                 byte_range(sin_tab, table_rows * (D / 2) * 4)};
    std::vector<Range> out_ranges;
    for (int i = 0; i < 3; ++i) {
        const int64_t tshape[4] = {B, S_l * c->P, heads[i] / c->P, D};
        if ((st = resolve_target(c, names[i], tags ? tags[i] : nullptr, outs ? outs[i] : nullptr,
                                 ULY_MODE_SCATTER, dtype, tshape, dsts[i])) != ULY_OK)
            return st;
        out_ranges.push_back(byte_range(dsts[i], int64_t(c->P) * tshape[0] * tshape[1] * tshape[2] * D * 2));
    }
    if ((st = check_overlaps(in_ranges, out_ranges)) != ULY_OK) return st;
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (out_ranges[i].overlaps(out_ranges[j]))
                return fail(ULY_E_OVERLAP, "targets %s and %s overlap", names[i], names[j]);
    if (c->host_only) return host_only_launch(c);
    if (M == 0) return ULY_OK;

    ProjArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = static_cast<const uint16_t *>(w_qkv);
    a.wn[0] = static_cast<const uint16_t *>(w_q);
    a.wn[1] = static_cast<const uint16_t *>(w_k);
    a.cos_tab = cos_tab;
    a.sin_tab = sin_tab;
    const int64_t S = S_l * c->P;
    for (int i = 0; i < 3; ++i) {
        const int64_t Hl = heads[i] / c->P;
        a.dst[i] = reinterpret_cast<uint16_t *>(dsts[i]);
        a.d_q[i] = B * S * Hl * D;
        a.d_b[i] = S * Hl * D;
        a.d_g[i] = Hl * D;
        a.hl[i] = FastDiv::make(uint32_t(Hl));
    }
    a.sl = FastDiv::make(uint32_t(S_l));
    a.bdiv = FastDiv::make(uint32_t(B));
    a.nhb = FastDiv::make(uint32_t(NHB));
    a.NH = uint32_t(NH);
    a.M = uint32_t(M);
    a.K = uint32_t(hidden);
    a.S_l = uint32_t(S_l);
    a.Hq = uint32_t(Hq);
    a.Hkv = uint32_t(Hkv);
    a.eps = eps;
    a.inv_D = 1.0f / float(D);
    const uint32_t blocks = uint32_t(tiles * NHB);
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    // a token operand beyond the Infinity Cache streams from HBM: prefetch its rows deeper
    const bool deep_b = c->proj_ring ? c->proj_ring == 3 : M * hidden * 2 > kCacheResidentBytes;
    if ((st = launch(c, ULY_K_PROJ, caller, [&] { launch_proj(a, dtype, blocks, deep_b, caller); })) != ULY_OK)
        return st;
    return mark_pending(c, caller);
}

uly_status uly_wait(uly_ctx *c, hipStream_t consumer) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (c->host_only) {
        c->pending.clear();
        return ULY_OK;
    }
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    for (auto &p : c->pending) {
        if (p.stream == consumer) continue;       // stream order already covers it
        hipError_t err = hipSuccess;
        hipEvent_t e = take_event(c->sync_pool, hipEventDisableTiming, err);
        if (!e) return poison(c, err, "hipEventCreate");
        c->sync_pool.push_back(e);                // reusable once the wait below is enqueued
        if ((err = hipEventRecord(e, p.stream)) != hipSuccess) return poison(c, err, "hipEventRecord");
        if ((err = hipStreamWaitEvent(consumer, e, 0)) != hipSuccess) return poison(c, err, "hipStreamWaitEvent");
    }
    c->pending.clear();
    return ULY_OK;
}

uly_status ulysses_gather_out(uly_ctx *c, const uly_tensor *o, const char *tag, void *out, hipStream_t caller) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    Operand x;
    if ((st = check_operand(o, "out", c->P, x)) != ULY_OK) return st;
    if (x.S % c->P != 0)
        return fail(ULY_E_INVAL, "gathered sequence %lld not divisible by world size %d", (long long)x.S, c->P);
    if (x.H > 1 && x.sh != x.D) return fail(ULY_E_INVAL, "out: heads must be packed (stride[2] == D)");
    const int64_t tshape[4] = {x.B, x.S / c->P, x.H * c->P, x.D};
    CopyBatch batch{};
    if (!x.empty()) {
        uint8_t *dst = nullptr;
        if ((st = resolve_target(c, "out", tag, out, ULY_MODE_GATHER, x.dtype, tshape, dst)) != ULY_OK) return st;
        std::vector<Range> in{x.range};
        std::vector<Range> outs{byte_range(dst, int64_t(c->P) * tshape[0] * tshape[1] * tshape[2] * tshape[3] * x.es)};
        if ((st = check_overlaps(in, outs)) != ULY_OK) return st;
        if ((st = plan_gather(x, c->P, dst, batch.p[0])) != ULY_OK) return st;
        batch.n = 1;
    }
    if ((st = finish_batch(batch)) != ULY_OK) return st;
    if (c->host_only) return host_only_launch(c);
    if (batch.n == 0) return ULY_OK;
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    return launch(c, ULY_K_GATHER, caller, [&] { launch_relayout(batch, caller); });
}

uly_status uly_exchange_chunks(uly_ctx *c, const void *x, void *y, int64_t chunk_bytes, hipStream_t stream) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (chunk_bytes < 0 || chunk_bytes % 16 != 0)
        return fail(ULY_E_INVAL, "chunk of %lld bytes is not a non-negative multiple of 16", (long long)chunk_bytes);
    const int64_t P = c->P, total_bytes = checked_prod({P, P, chunk_bytes});
    if (total_bytes < 0 || total_bytes / 16 >= kMaxVecs) return fail(ULY_E_UNSUPPORTED, "too large for one launch");
    CopyBatch batch{};
    if (total_bytes > 0) {
        if (!x || !y || !aligned16(x) || !aligned16(y)) return fail(ULY_E_INVAL, "x, y null or not 16-byte aligned");
        if (byte_range(x, total_bytes).overlaps(byte_range(y, total_bytes)))
            return fail(ULY_E_OVERLAP, "x and y overlap");
        // y[q][r][:] = x[r][q][:], iterated in destination order (q, r)
        const int64_t n[4] = {P, P, 1, 1}, ss[4] = {chunk_bytes, P * chunk_bytes, 0, 0},
                      ds[4] = {P * chunk_bytes, chunk_bytes, 0, 0};
        fill_plan(batch.p[0], static_cast<const uint8_t *>(x), static_cast<uint8_t *>(y), n, ss, ds,
                  chunk_bytes / 16, total_bytes / 16);
        batch.n = 1;
    }
    if ((st = finish_batch(batch)) != ULY_OK) return st;
    if (c->host_only) return host_only_launch(c);
    if (batch.n == 0) return ULY_OK;
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    return launch(c, ULY_K_SCATTER, stream, [&] { launch_relayout(batch, stream); });
}

// ---- sequence padding ------------------------------------------------------

static uly_status rowmap_common(uly_ctx *c, const void *src, int dtype, int64_t row_elems, void *dst,
                                int64_t src_rows, int64_t dst_rows, RowMapArgs &a) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (!valid_dtype(dtype)) return fail(ULY_E_DTYPE, "bad dtype %d", dtype);
    const int64_t es = elem_size(dtype);
    if (row_elems < 1 || row_elems > kMaxExtent || (row_elems * es) % 16 != 0)
        return fail(ULY_E_INVAL, "row of %lld elements is not a positive multiple of 16 bytes",
                    (long long)row_elems);
    if (src_rows < 0 || dst_rows < 0) return fail(ULY_E_INVAL, "negative or too large extent");
    const int64_t vpr = row_elems * es / 16;
    const int64_t total = checked_prod({dst_rows, vpr}), src_total = checked_prod({src_rows, vpr});
    if (total < 0 || src_total < 0 || total >= kMaxVecs || src_total >= kMaxVecs)
        return fail(ULY_E_UNSUPPORTED, "too large for one launch");
    if (total > 0) {
        if (!dst || !aligned16(dst)) return fail(ULY_E_INVAL, "destination null or not 16-byte aligned");
        if (src_rows > 0 && (!src || !aligned16(src))) return fail(ULY_E_INVAL, "source null or not 16-byte aligned");
        if (byte_range(src, src_rows * row_elems * es).overlaps(byte_range(dst, dst_rows * row_elems * es)))
            return fail(ULY_E_OVERLAP, "source and destination overlap");
    }
    a = RowMapArgs{};
    a.src = static_cast<const uint8_t *>(src);
    a.dst = static_cast<uint8_t *>(dst);
    a.vpr = FastDiv::make(uint32_t(vpr));
    a.total = uint32_t(total);
    return ULY_OK;
}

static uly_status rowmap_launch(uly_ctx *c, const RowMapArgs &a, int rkind, int pkind, hipStream_t s) {
    if (c->host_only) return host_only_launch(c);
    if (a.total == 0) return ULY_OK;
    DeviceGuard g(c->device);
    if (g.err != hipSuccess) return poison(c, g.err, "hipSetDevice");
    return launch(c, pkind, s, [&] { launch_rowmap(a, rkind, s); });
}

uly_status uly_seq_pad_shard(uly_ctx *c, const void *full, int dtype, int64_t B, int64_t S, int64_t row_elems,
                             int64_t S_l, void *x, hipStream_t stream) {
    if (c && (B < 0 || S < 0 || S_l < 0 || S_l > kMaxExtent || int64_t(c->P) * S_l < S))
        return fail(ULY_E_INVAL, "need B, S >= 0 and P*S_l >= S");
    RowMapArgs a;
    // an overflowing product comes back as -1, which rowmap_common rejects
    uly_status st = rowmap_common(c, full, dtype, row_elems, x, checked_prod({B, S}),
                                  checked_prod({c ? c->P : 0, B, S_l}), a);
    if (st != ULY_OK) return st;
    a.f0 = FastDiv::make(uint32_t(S_l));
    a.f1 = FastDiv::make(uint32_t(B));
    a.B_or_N = uint32_t(B);
    a.S = uint32_t(S);
    a.S_l = uint32_t(S_l);
    return rowmap_launch(c, a, kPadShard, ULY_K_PAD, stream);
}

uly_status uly_seq_unshard_trim(uly_ctx *c, const void *x, int dtype, int64_t B, int64_t S, int64_t row_elems,
                                int64_t S_l, void *full, hipStream_t stream) {
    if (c && (B < 0 || S < 0 || S_l < 0 || S_l > kMaxExtent || int64_t(c->P) * S_l < S))
        return fail(ULY_E_INVAL, "need B, S >= 0 and P*S_l >= S");
    RowMapArgs a;
    uly_status st = rowmap_common(c, x, dtype, row_elems, full, checked_prod({c ? c->P : 0, B, S_l}),
                                  checked_prod({B, S}), a);
    if (st != ULY_OK) return st;
    a.f0 = FastDiv::make(uint32_t(S));
    a.f2 = FastDiv::make(uint32_t(S_l));
    a.B_or_N = uint32_t(B);
    a.S = uint32_t(S);
    a.S_l = uint32_t(S_l);
    return rowmap_launch(c, a, kUnshardTrim, ULY_K_PAD, stream);
}

// ---- spatial ---------------------------------------------------------------

static uly_status spatial_dims(uly_ctx *c, int64_t N, int64_t Hh, int64_t W, int64_t halo, int64_t &hmax) {
    if (!c) return fail(ULY_E_INVAL, "null context");
    if (N < 0 || Hh < 1 || W < 1 || halo < 0 || N > kMaxExtent || Hh > kMaxExtent || W > kMaxExtent)
        return fail(ULY_E_INVAL, "bad spatial extents");
    if (Hh < c->P) return fail(ULY_E_INVAL, "height %lld smaller than world size %d", (long long)Hh, c->P);
    hmax = (Hh + c->P - 1) / c->P;
    if (halo > hmax) return fail(ULY_E_INVAL, "halo larger than a shard");
    return ULY_OK;
}

static void spatial_fill(RowMapArgs &a, int P, int64_t N, int64_t Hh, int64_t hmax, int64_t halo) {
    a.B_or_N = uint32_t(N);
    a.S = uint32_t(Hh);
    a.S_l = uint32_t(hmax);
    a.halo = uint32_t(halo);
    a.base_h = uint32_t(Hh / P);
    a.extra_h = uint32_t(Hh % P);
}

uly_status uly_spatial_split_halo(uly_ctx *c, const void *full, int dtype, int64_t N, int64_t Hh, int64_t W,
                                  int64_t halo, void *shards, hipStream_t stream) {
    int64_t hmax = 0;
    uly_status st = spatial_dims(c, N, Hh, W, halo, hmax);
    if (st != ULY_OK) return st;
    RowMapArgs a;
    const int64_t R2 = hmax + 2 * halo;
    if ((st = rowmap_common(c, full, dtype, W, shards, checked_prod({N, Hh}), checked_prod({c->P, N, R2}), a)) !=
        ULY_OK)
        return st;
    a.f0 = FastDiv::make(uint32_t(R2));
    a.f1 = FastDiv::make(uint32_t(N));
    spatial_fill(a, c->P, N, Hh, hmax, halo);
    return rowmap_launch(c, a, kSplitHalo, ULY_K_SPATIAL, stream);
}

uly_status uly_spatial_gather_stacked(uly_ctx *c, const void *shards, int dtype, int64_t N, int64_t Hh,
                                      int64_t W, int64_t halo, void *stacked, hipStream_t stream) {
    int64_t hmax = 0;
    uly_status st = spatial_dims(c, N, Hh, W, halo, hmax);
    if (st != ULY_OK) return st;
    RowMapArgs a;
    const int64_t R2 = hmax + 2 * halo;
    if ((st = rowmap_common(c, shards, dtype, W, stacked, checked_prod({c->P, N, R2}), checked_prod({c->P, N, hmax}),
                            a)) != ULY_OK)
        return st;
    a.f0 = FastDiv::make(uint32_t(hmax));
    a.f1 = FastDiv::make(uint32_t(N));
    spatial_fill(a, c->P, N, Hh, hmax, halo);
    return rowmap_launch(c, a, kGatherStacked, ULY_K_SPATIAL, stream);
}

uly_status uly_spatial_trim_concat(uly_ctx *c, const void *stacked, int dtype, int64_t N, int64_t Hh, int64_t W,
                                   void *full, hipStream_t stream) {
    int64_t hmax = 0;
    uly_status st = spatial_dims(c, N, Hh, W, 0, hmax);
    if (st != ULY_OK) return st;
    RowMapArgs a;
    if ((st = rowmap_common(c, stacked, dtype, W, full, checked_prod({c->P, N, hmax}), checked_prod({N, Hh}), a)) !=
        ULY_OK)
        return st;
    a.f0 = FastDiv::make(uint32_t(Hh));
    a.f2 = FastDiv::make(uint32_t(Hh / c->P + 1));
    a.f3 = FastDiv::make(uint32_t(Hh / c->P));
    spatial_fill(a, c->P, N, Hh, hmax, 0);
    return rowmap_launch(c, a, kTrimConcat, ULY_K_SPATIAL, stream);
}

// ---- rotary tables (host) ----------------------------------------------------

uly_status uly_rope_table_1d(float *cos_out, float *sin_out, int64_t rows, int64_t real_rows, int64_t D,
                             double theta) {
    if (!cos_out || !sin_out || rows < 0 || real_rows < 0 || D < 2 || D % 2 || !(theta > 0) ||
        checked_prod({rows, D}) < 0)
        return fail(ULY_E_INVAL, "bad rope table arguments");
    const int64_t half = D / 2;
    std::vector<double> inv_freq(half);
    for (int64_t j = 0; j < half; ++j) inv_freq[j] = std::pow(theta, -2.0 * double(j) / double(D));
    for (int64_t g = 0; g < rows; ++g)
        for (int64_t j = 0; j < half; ++j) {
            const bool real = g < real_rows;
            const double ang = double(g) * inv_freq[j];
            cos_out[g * half + j] = real ? float(std::cos(ang)) : 1.0f;
            sin_out[g * half + j] = real ? float(std::sin(ang)) : 0.0f;
        }
    return ULY_OK;
}

uly_status uly_rope_table_3d(float *cos_out, float *sin_out, int64_t rows, int64_t real_rows, int64_t D,
                             int64_t grid_h, int64_t grid_w, int64_t n_t, int64_t n_h, int64_t n_w, double theta) {
    if (!cos_out || !sin_out || rows < 0 || real_rows < 0 || D < 2 || D % 2 || grid_h < 1 || grid_w < 1 ||
        n_t < 0 || n_h < 0 || n_w < 0 || n_t + n_h + n_w > D / 2 || !(theta > 0) || checked_prod({rows, D}) < 0 ||
        checked_prod({grid_h, grid_w}) < 0)
        return fail(ULY_E_INVAL, "bad 3-D rope table arguments");
    const int64_t half = D / 2;
    const int64_t band_start[3] = {0, n_t, n_t + n_h};
    const int64_t band_len[3] = {n_t, n_h, n_w};
    for (int64_t g = 0; g < rows; ++g) {
        const int64_t coord[3] = {g / (grid_h * grid_w), (g / grid_w) % grid_h, g % grid_w};
        for (int64_t j = 0; j < half; ++j) {
            cos_out[g * half + j] = 1.0f;
            sin_out[g * half + j] = 0.0f;
        }
        if (g >= real_rows) continue;
        for (int axis = 0; axis < 3; ++axis)
            for (int64_t k = 0; k < band_len[axis]; ++k) {
                const double ang =
                    double(coord[axis]) * std::pow(theta, -2.0 * double(k) / double(2 * band_len[axis]));
                cos_out[g * half + band_start[axis] + k] = float(std::cos(ang));
                sin_out[g * half + band_start[axis] + k] = float(std::sin(ang));
            }
    }
    return ULY_OK;
}

// ---- measurement and test hooks ------------------------------------------------

uly_status uly_profile_enable(uly_ctx *c, int kind_mask, int every) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (every < 1) return fail(ULY_E_INVAL, "every must be >= 1");
    c->profile_mask = kind_mask & ((1 << ULY_K_COUNT) - 1);
    c->profile_every = every;
    for (auto &n : c->profile_seen) n = 0;
    return ULY_OK;
}

uly_status uly_profile_read(uly_ctx *c, int kind, double *total_ms, int64_t *launches) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (kind < 0 || kind >= ULY_K_COUNT || !total_ms || !launches) return fail(ULY_E_INVAL, "bad arguments");
    double sum = 0;
    int64_t n = 0;
    for (auto &r : c->prof) {
        if (r.kind != kind) continue;
        if (r.ms < 0) {
            hipError_t err = hipEventSynchronize(r.stop);
            float ms = 0;
            if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.start, r.stop);
            if (err != hipSuccess) return poison(c, err, "reading timing events");
            r.ms = ms;
        }
        sum += r.ms;
        ++n;
    }
    *total_ms = sum;
    *launches = n;
    return ULY_OK;
}

uly_status uly_profile_reset(uly_ctx *c) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    for (auto &r : c->prof) {
        if (r.ms < 0) (void)hipEventSynchronize(r.stop);
        c->timing_pool.push_back(r.start);
        c->timing_pool.push_back(r.stop);
    }
    c->prof.clear();
    return ULY_OK;
}

uly_status uly_get_stats(uly_ctx *c, uly_stats *out) {
    if (!c || !out) return fail(ULY_E_INVAL, "null argument");
    *out = c->stats;
    return ULY_OK;
}

uly_status uly_comm_stream(uly_ctx *c, hipStream_t *out) {
    if (!c || !out) return fail(ULY_E_INVAL, "null argument");
    *out = c->comm;
    return ULY_OK;
}

uly_status uly_set_route(uly_ctx *c, int route) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (route != ULY_ROUTE_KERNEL && route != ULY_ROUTE_COPY_ENGINE && route != ULY_ROUTE_CALLER)
        return fail(ULY_E_INVAL, "bad route %d", route);
    c->route = route;
    return ULY_OK;
}

uly_status uly_debug_fail_launch(uly_ctx *c, int after) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    c->fail_after = after < 0 ? -1 : after;
    return ULY_OK;
}

uly_status uly_debug_proj_ring(uly_ctx *c, int depth) {
    uly_status st = ctx_ok(c);
    if (st != ULY_OK) return st;
    if (depth != 0 && depth != 2 && depth != 3) return fail(ULY_E_INVAL, "ring depth %d: 0, 2 or 3", depth);
    c->proj_ring = depth;
    return ULY_OK;
}

}  // extern "C"
