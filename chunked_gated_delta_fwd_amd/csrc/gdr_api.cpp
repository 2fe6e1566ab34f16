// Host side of the C ABI declared in include/gdr.h: descriptor validation,
// launch planning from shapes only, stream-ordered workspace, error text.
//
// Validation rules follow the pages' integration lessons: NULL strides mean
// compact row-major ("Findings from integrating FlashQLA's Blackwell GDN
// kernels into a JAX trainer", item 3), length-0 segments are legal anywhere
// (item 2), chunk indices come from the cu_seqlens content on the device every
// call and nothing is cached by tensor identity (item 1).
#include "gdr.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "gdr_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return GDR_OK;
}

size_t dtype_size(int32_t dt) { return dt == GDR_F32 ? 4 : dt == GDR_BF16 ? 2 : dt == GDR_I32 ? 4 : 0; }

const char *dtype_name(int32_t dt) {
    return dt == GDR_F32 ? "f32" : dt == GDR_BF16 ? "bf16" : dt == GDR_I32 ? "i32" : "?";
}

struct Span {
    uintptr_t lo = 0, hi = 0;   // [lo, hi) bytes; empty when lo == hi
};

// Checks rank, non-negative extents, compact strides and the data pointer.
int check_tensor(const gdr_tensor *t, const char *name, int ndim, int64_t *numel, size_t align) {
    if (!t) return fail(GDR_EINVAL, "%s: descriptor is NULL", name);
    if (t->ndim != ndim) return fail(GDR_ESHAPE, "%s: expected %d dimensions, got %d", name, ndim, t->ndim);
    if (ndim > 0 && !t->shape) return fail(GDR_EINVAL, "%s: shape pointer is NULL", name);
    if (dtype_size(t->dtype) == 0) return fail(GDR_EDTYPE, "%s: unknown dtype %d", name, t->dtype);
    int64_t n = 1;
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0) return fail(GDR_ESHAPE, "%s: negative extent in dimension %d", name, i);
        if (t->shape[i] > 0 && n > (INT64_MAX / 16) / t->shape[i])
            return fail(GDR_ESHAPE, "%s: too many elements", name);
        n *= t->shape[i];
    }
    if (t->strides) {
        int64_t expect = 1;
        for (int i = ndim - 1; i >= 0; --i) {
            if (t->shape[i] != 1 && t->strides[i] != expect)
                return fail(GDR_ESTRIDE,
                            "%s: strides must be compact row-major (dimension %d has stride %lld, expected %lld)",
                            name, i, (long long)t->strides[i], (long long)expect);
            expect *= t->shape[i];
        }
    }
    if (n > 0 && !t->data) return fail(GDR_EINVAL, "%s: data pointer is NULL", name);
    if (n > 0 && (reinterpret_cast<uintptr_t>(t->data) % align) != 0)
        return fail(GDR_EINVAL, "%s: data pointer must be %zu-byte aligned", name, align);
    *numel = n;
    return GDR_OK;
}

Span span_of(const gdr_tensor *t, int64_t numel) {
    Span s;
    if (t && t->data && numel > 0) {
        s.lo = reinterpret_cast<uintptr_t>(t->data);
        s.hi = s.lo + static_cast<uintptr_t>(numel) * dtype_size(t->dtype);
    }
    return s;
}

bool overlap(const Span &a, const Span &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool shape_is(const gdr_tensor *t, std::initializer_list<int64_t> s) {
    int i = 0;
    for (int64_t e : s)
        if (t->shape[i++] != e) return false;
    return true;
}

std::string shape_str(const gdr_tensor *t) {
    std::string s = "[";
    for (int i = 0; i < t->ndim; ++i) {
        if (i) s += ", ";
        s += std::to_string(static_cast<long long>(t->shape[i]));
    }
    return s + "]";
}

// Validates a forward call and fills the plan (shapes only, no device access).
// The backward pass reuses it for its inputs: there `o` is the incoming
// gradient do (named `o_name`, an input, so not checked for overlaps).
int plan_fwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
             const gdr_tensor *beta, const gdr_tensor *cu, const gdr_tensor *h0, const gdr_tensor *o,
             const gdr_tensor *ht, float scale, gdr_launch_plan *p, const char *o_name = "o") {
    const bool o_out = std::strcmp(o_name, "o") == 0;
    int64_t nq, nk, nv, ng, nb, no, ncu = 0, nh0 = 0, nht = 0;
    int rc;
    if ((rc = check_tensor(q, "q", 4, &nq, 16))) return rc;
    if ((rc = check_tensor(k, "k", 4, &nk, 16))) return rc;
    if ((rc = check_tensor(v, "v", 4, &nv, 16))) return rc;
    if ((rc = check_tensor(g, "g", 3, &ng, 4))) return rc;
    if ((rc = check_tensor(beta, "beta", 3, &nb, 4))) return rc;
    if ((rc = check_tensor(o, o_name, 4, &no, 16))) return rc;
    if (cu && (rc = check_tensor(cu, "cu_seqlens", 1, &ncu, 4))) return rc;
    if (h0 && (rc = check_tensor(h0, "h0", 4, &nh0, 4))) return rc;
    if (ht && (rc = check_tensor(ht, "ht", 4, &nht, 4))) return rc;

    if (q->dtype != GDR_BF16 && q->dtype != GDR_F32)
        return fail(GDR_EDTYPE, "q: dtype must be bf16 or f32, got %s", dtype_name(q->dtype));
    if (k->dtype != q->dtype || v->dtype != q->dtype || o->dtype != q->dtype)
        return fail(GDR_EDTYPE, "q, k, v and %s must share one dtype (q is %s)", o_name, dtype_name(q->dtype));
    if (g->dtype != GDR_BF16 && g->dtype != GDR_F32)
        return fail(GDR_EDTYPE, "g: dtype must be bf16 or f32, got %s", dtype_name(g->dtype));
    if (beta->dtype != g->dtype) return fail(GDR_EDTYPE, "beta must have the dtype of g");
    if (cu && cu->dtype != GDR_I32) return fail(GDR_EDTYPE, "cu_seqlens: dtype must be i32");
    if (h0 && h0->dtype != GDR_F32) return fail(GDR_EDTYPE, "h0: dtype must be f32");
    if (ht && ht->dtype != GDR_F32) return fail(GDR_EDTYPE, "ht: dtype must be f32");

    const int64_t B = q->shape[0], T = q->shape[1], Hk = q->shape[2], dk = q->shape[3];
    const int64_t Hv = v->shape[2], dv = v->shape[3];
    if (!shape_is(k, {B, T, Hk, dk}))
        return fail(GDR_ESHAPE, "k: shape %s must equal q's %s", shape_str(k).c_str(), shape_str(q).c_str());
    if (v->shape[0] != B || v->shape[1] != T)
        return fail(GDR_ESHAPE, "v: shape %s must be [B, T, Hv, dv] with q's B, T", shape_str(v).c_str());
    if (!shape_is(o, {B, T, Hv, dv}))
        return fail(GDR_ESHAPE, "%s: shape %s must equal v's %s", o_name, shape_str(o).c_str(), shape_str(v).c_str());
    if (!shape_is(g, {B, T, Hv}) || !shape_is(beta, {B, T, Hv}))
        return fail(GDR_ESHAPE, "g and beta must be [B, T, Hv] = [%lld, %lld, %lld]", (long long)B,
                    (long long)T, (long long)Hv);
    if (dk != 64 && dk != 128) return fail(GDR_ESHAPE, "dk must be 64 or 128, got %lld", (long long)dk);
    if (dv != 64 && dv != 128) return fail(GDR_ESHAPE, "dv must be 64 or 128, got %lld", (long long)dv);
    if (Hk < 1 || Hv < 1) return fail(GDR_ESHAPE, "head counts must be positive");
    if (Hv % Hk != 0)
        return fail(GDR_ESHAPE, "Hv (%lld) must be a multiple of Hk (%lld)", (long long)Hv, (long long)Hk);
    if (Hv > 65536) return fail(GDR_ESHAPE, "too many v-heads");

    int64_t N;
    if (cu) {
        if (B != 1) return fail(GDR_ESHAPE, "cu_seqlens requires B == 1 (got B = %lld)", (long long)B);
        if (cu->shape[0] < 1) return fail(GDR_ESHAPE, "cu_seqlens must hold at least one offset");
        N = cu->shape[0] - 1;
    } else {
        N = B;
    }
    if (h0 && !shape_is(h0, {N, Hv, dk, dv}))
        return fail(GDR_ESHAPE, "h0: shape %s must be [N, Hv, dk, dv] = [%lld, %lld, %lld, %lld]",
                    shape_str(h0).c_str(), (long long)N, (long long)Hv, (long long)dk, (long long)dv);
    if (ht && !shape_is(ht, {N, Hv, dk, dv}))
        return fail(GDR_ESHAPE, "ht: shape %s must be [N, Hv, dk, dv] = [%lld, %lld, %lld, %lld]",
                    shape_str(ht).c_str(), (long long)N, (long long)Hv, (long long)dk, (long long)dv);
    if (!std::isfinite(scale)) return fail(GDR_EINVAL, "scale must be finite");
    if (N * Hv > 0x7FFFFFFFLL) return fail(GDR_ESHAPE, "N * Hv exceeds the launch grid limit");
    if (B * T > 0x7FFFFFFFLL) return fail(GDR_ESHAPE, "B * T exceeds 2^31 - 1 tokens");

    const Span so = span_of(o, no), sht = span_of(ht, nht);
    const Span ins[] = {span_of(q, nq), span_of(k, nk), span_of(v, nv), span_of(g, ng),
                        span_of(beta, nb), span_of(cu, ncu), span_of(h0, nh0)};
    for (const Span &s : ins) {
        if (o_out && overlap(so, s)) return fail(GDR_EALIAS, "o overlaps an input");
        if (overlap(sht, s)) return fail(GDR_EALIAS, "ht overlaps an input");
    }
    if (overlap(so, sht)) return fail(GDR_EALIAS, "o and ht overlap");

    std::memset(p, 0, sizeof(*p));
    p->n_seq = N;
    p->total_tokens = B * T;
    p->nt_max = (B * T + gdr::kChunk - 1) / gdr::kChunk + N;
    p->hk = static_cast<int32_t>(Hk);
    p->hv = static_cast<int32_t>(Hv);
    p->d = static_cast<int32_t>(dk);
    p->dv = static_cast<int32_t>(dv);
    p->in_dtype = q->dtype;
    p->gate_dtype = g->dtype;
    p->varlen = cu ? 1 : 0;
    p->has_h0 = h0 ? 1 : 0;
    p->has_ht = ht ? 1 : 0;
    p->grid_fwd = N * Hv;
    const bool f32 = q->dtype == GDR_F32;   // f32 inputs: the token-serial fp32 kernel
    p->block_fwd = f32 ? gdr::kFwdF32Threads : gdr::kFwdThreads;
    p->lds_fwd = f32 ? gdr::fwd_f32_lds_bytes(static_cast<int>(dk), static_cast<int>(dv))
                     : gdr::fwd_lds_bytes(static_cast<int>(dk));
    p->workspace_bytes = cu ? 4 * N + 16 : 0;
    return GDR_OK;
}

// gfx950 check for the current device, remembered per device ordinal.
int check_device() {
    static int state[64];   // 0 unknown, 1 gfx950, -1 other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GDR_EDEVICE, "hipGetDevice failed");
    if (dev >= 0 && dev < 64 && state[dev] == 1) return GDR_OK;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(GDR_EDEVICE, "hipGetDeviceProperties failed for device %d", dev);
    const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) state[dev] = good ? 1 : -1;
    if (!good) return fail(GDR_EDEVICE, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
    return GDR_OK;
}

// Library-owned device workspaces, reused across calls.  On this runtime
// freeing a stream-ordered allocation (hipFreeAsync) blocks the calling
// thread until the stream has caught up, which serialised the host with the
// GPU at every call.  Instead each device keeps a ring of buffers that are
// never freed while in use: a call takes the next slot of the ring (or the
// one large slot, for the backward's multi-GB workspace), makes its stream
// wait on the GPU for the slot's previous user (an event recorded after that
// user's last kernel, so reuse is ordered across streams without a host
// wait), and records the event again after its own kernels.  Slots are
// indexed by a counter, never by stream or tensor identity.
//
// The whole ring is created by the first call on a device: one allocation
// holding all slots (at least kRingSlot bytes each) and all events, so later
// calls allocate nothing.  A request larger than a slot regrows the whole ring
// once (every slot's previous user is waited for first).  Everything is kept
// until gdr_free_workspaces or the end of the process.
int launch_error(hipError_t e, const char *what) {
    return fail(GDR_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kRing = 8;
constexpr size_t kRingSlot = 1u << 20;
constexpr int kMaxDevices = 64;
struct WsSlot {
    std::mutex mu;
    hipEvent_t ev = nullptr;
    bool used = false;
};
struct WsDevice {
    // mu guards next, block and cap; a regrow also holds every slot's lock,
    // so a thread holding one slot's lock reads block and cap unchanged.
    std::mutex mu;
    unsigned next = 0;
    unsigned char *block = nullptr;   // kRing slots of cap bytes
    size_t cap = 0;
    WsSlot ring[kRing];
    WsSlot big;
    void *big_ptr = nullptr;
    size_t big_cap = 0;
};
WsDevice g_ws[kMaxDevices];

size_t round_mib(size_t x) { return (x + 0xFFFFF) & ~static_cast<size_t>(0xFFFFF); }

// (Re)creates the ring of device D with slots of at least `bytes`; the caller
// holds D.mu and no slot lock.
int ring_grow(WsDevice &D, size_t bytes) {
    std::unique_lock<std::mutex> locks[kRing];
    for (int i = 0; i < kRing; ++i) locks[i] = std::unique_lock<std::mutex>(D.ring[i].mu);
    for (WsSlot &s : D.ring)
        if (s.used) {
            (void)hipEventSynchronize(s.ev);
            s.used = false;
        }
    if (D.block) (void)hipFree(D.block);
    D.block = nullptr;
    D.cap = 0;
    const size_t cap = round_mib(bytes > kRingSlot ? bytes : kRingSlot);
    void *p = nullptr;
    const hipError_t e = hipMalloc(&p, cap * kRing);
    if (e != hipSuccess) return fail(GDR_ENOMEM, "workspace ring of %zu bytes: %s", cap * kRing, hipGetErrorString(e));
    for (WsSlot &s : D.ring)
        if (!s.ev && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) {
            s.ev = nullptr;
            (void)hipFree(p);
            return fail(GDR_ENOMEM, "workspace event could not be created");
        }
    D.block = static_cast<unsigned char *>(p);
    D.cap = cap;
    return GDR_OK;
}

// Holds one slot from acquire() to release(); the slot's lock is kept in
// between so that its event is recorded before anyone else can take it.
class WsLease {
  public:
    int acquire(size_t bytes, bool big, hipStream_t stream, void **out) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return fail(GDR_EDEVICE, "no current device");
        WsDevice &D = g_ws[dev];
        WsSlot *s;
        void *ptr;
        if (big) {
            s = &D.big;
            lock_ = std::unique_lock<std::mutex>(s->mu);
            if (!s->ev && hipEventCreateWithFlags(&s->ev, hipEventDisableTiming) != hipSuccess) {
                s->ev = nullptr;
                return fail(GDR_ENOMEM, "workspace event could not be created");
            }
            if (D.big_cap < bytes) {
                if (D.big_ptr) {
                    if (s->used) (void)hipEventSynchronize(s->ev);
                    (void)hipFree(D.big_ptr);
                    D.big_ptr = nullptr;
                    D.big_cap = 0;
                    s->used = false;
                }
                const size_t want = round_mib(bytes > 65536 ? bytes : 65536);
                const hipError_t e = hipMalloc(&D.big_ptr, want);
                if (e != hipSuccess) {
                    D.big_ptr = nullptr;
                    return fail(GDR_ENOMEM, "workspace of %zu bytes: %s", want, hipGetErrorString(e));
                }
                D.big_cap = want;
            }
            ptr = D.big_ptr;
        } else {
            unsigned idx;
            {
                std::lock_guard<std::mutex> g(D.mu);
                if (!D.block || D.cap < bytes) {
                    const int rc = ring_grow(D, bytes);
                    if (rc) return rc;
                }
                idx = D.next++ % kRing;
            }
            s = &D.ring[idx];
            lock_ = std::unique_lock<std::mutex>(s->mu);
            ptr = D.block + static_cast<size_t>(idx) * D.cap;
        }
        if (s->used && hipEventQuery(s->ev) != hipSuccess) {
            const hipError_t e = hipStreamWaitEvent(stream, s->ev, 0);
            if (e != hipSuccess) return launch_error(e, "workspace wait");
        }
        slot_ = s;
        stream_ = stream;
        *out = ptr;
        return GDR_OK;
    }
    // After the call's last kernel that touches the workspace (also on error
    // paths: whatever was enqueued is then ordered before the next user).
    int release() {
        if (!slot_) return GDR_OK;
        const hipError_t e = hipEventRecord(slot_->ev, stream_);
        if (e == hipSuccess) slot_->used = true;
        slot_ = nullptr;
        lock_.unlock();
        return e == hipSuccess ? GDR_OK : launch_error(e, "workspace release");
    }
    ~WsLease() { (void)release(); }

  private:
    WsSlot *slot_ = nullptr;
    hipStream_t stream_ = nullptr;
    std::unique_lock<std::mutex> lock_;
};

// Debug and test options (gdr_debug_set).  The cu_seqlens content check can
// also be switched on for the whole process with GDR_DEBUG_CHECK_CU=1.
std::atomic<int> g_check_cu{[] {
    const char *e = std::getenv("GDR_DEBUG_CHECK_CU");
    return (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
}()};
std::atomic<int64_t> g_fail_launches{0};
std::atomic<int32_t> g_spin_max{gdr::kSpinDefault};

// True when the test hook says this launch is to fail (consumes one).
bool forced_failure() {
    int64_t n = g_fail_launches.load(std::memory_order_relaxed);
    while (n > 0)
        if (g_fail_launches.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) return true;
    return false;
}
hipError_t launch_or_fail(hipError_t (*launch)(const gdr::FwdArgs &, hipStream_t), const gdr::FwdArgs &a,
                          hipStream_t stream) {
    return forced_failure() ? hipErrorLaunchFailure : launch(a, stream);
}

// Fills the device status pointer and spin limit every forward-kernel launch needs.
int fwd_defaults(gdr::FwdArgs &a) {
    const hipError_t e = gdr::device_buffers(&a.status, nullptr);
    if (e != hipSuccess) return fail(GDR_EDEVICE, "device status word: %s", hipGetErrorString(e));
    a.spin_max = g_spin_max.load(std::memory_order_relaxed);
    return GDR_OK;
}

// With the cu_seqlens check on: checks the content on the device, waits for
// the stream and reports the first violated precondition (GDR_EINVAL).
// `result` is 16 bytes of device workspace owned by the call.
int check_cu_content(const int32_t *cu, int64_t n_seq, int64_t total, int32_t *result, hipStream_t stream) {
    if (!g_check_cu.load(std::memory_order_relaxed)) return GDR_OK;
    hipError_t e = gdr::launch_check_cu(cu, n_seq, total, result, stream);
    if (e != hipSuccess) return launch_error(e, "cu_seqlens check kernel");
    int32_t r[4];
    if ((e = hipMemcpyAsync(r, result, sizeof(r), hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (e = hipStreamSynchronize(stream)) != hipSuccess)
        return launch_error(e, "cu_seqlens check");
    switch (r[0]) {
    case 0: return GDR_OK;
    case 1: return fail(GDR_EINVAL, "cu_seqlens: cu[0] must be 0, got %d", r[2]);
    case 2: return fail(GDR_EINVAL, "cu_seqlens: offsets must not decrease (cu[%d] = %d > cu[%d] = %d)", r[1], r[2],
                        r[1] + 1, r[3]);
    default: return fail(GDR_EINVAL, "cu_seqlens: cu[N] = cu[%d] = %d must equal the %d tokens", r[1], r[2], r[3]);
    }
}

// Machines of the dispatch-order model for a forward launch (kda: the
// per-channel-gate kernel): work-groups resident at once divided by the
// v-heads of a sequence (each XCD gets Hv/8 heads of every sequence, so Hv
// must split over the 8 XCDs), or 0 when the packed order does not apply.
// Occupancy is queried once per device and kernel variant.
int order_groups(const gdr::FwdArgs &a, bool kda = false) {
    if (!a.in_bf16) return 0;   // f32 inputs run the token-serial kernel: longest first is enough
    static std::mutex mu;
    static int cache[64][2][2][2][2][2];   // slots + 1; 0 unknown
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int &entry = cache[dev][kda ? 1 : 0][a.d == 64 ? 0 : 1][a.dv == 64 ? 0 : 1][a.in_bf16 ? 1 : 0][a.gate_bf16 ? 1 : 0];
    int slots = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (entry == 0) {
            int s = 0;
            const hipError_t e = kda ? gdr::kda_slots(a.d, a.in_bf16, a.gate_bf16, &s)
                                     : gdr::fwd_slots(a.d, a.dv, a.in_bf16, a.gate_bf16, &s);
            entry = e == hipSuccess ? s + 1 : 1;
        }
        slots = entry - 1;
    }
    if (a.hv % 8 != 0 || slots <= 0 || slots % a.hv != 0) return 0;
    const int groups = slots / a.hv;
    return (groups >= 2 && groups <= 16 && a.n_seq > groups && a.n_seq <= 64) ? groups : 0;
}


// The forward launch shared by gdr_chunk_fwd, gdr_chunk_fwd_checkpoints(_n)
// and gdr_chunk_fwd_noalloc (hck: checkpoint states every `every` tokens, or NULL).
int run_fwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
            const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
            const gdr_tensor *o, const gdr_tensor *ht, const gdr_tensor *hck, float scale,
            hipStream_t stream, bool noalloc = false, int64_t every = gdr::kChunk) {
    gdr_launch_plan p;
    int rc = plan_fwd(q, k, v, g, beta, cu_seqlens, h0, o, ht, scale, &p);
    if (rc) return rc;
    int64_t rows = 0;
    if (hck) {
        if (every < 16 || every % 16 != 0 || every > (int64_t{1} << 30))
            return fail(GDR_EINVAL, "every_n: %lld must be a positive multiple of 16 (at most 2^30)", (long long)every);
        int64_t nck;
        if ((rc = check_tensor(hck, "h_chunks", 4, &nck, 4))) return rc;
        if (hck->dtype != GDR_F32) return fail(GDR_EDTYPE, "h_chunks: dtype must be f32");
        const int64_t T = q->shape[1];
        rows = cu_seqlens ? (p.total_tokens + every - 1) / every + p.n_seq : q->shape[0] * ((T + every - 1) / every);
        if (!shape_is(hck, {rows, p.hv, p.d, p.dv}))
            return fail(GDR_ESHAPE, "h_chunks: shape %s must be [%lld, Hv, dk, dv] = [%lld, %d, %d, %d] for pieces of %lld tokens",
                        shape_str(hck).c_str(), (long long)rows, (long long)rows, p.hv, p.d, p.dv, (long long)every);
        const Span sck = span_of(hck, nck);
        const gdr_tensor *others[] = {q, k, v, g, beta, cu_seqlens, h0, o, ht};
        for (const gdr_tensor *t : others) {
            if (!t) continue;
            int64_t nt = 1;
            for (int i = 0; i < t->ndim; ++i) nt *= t->shape[i];
            if (overlap(sck, span_of(t, nt))) return fail(GDR_EALIAS, "h_chunks overlaps another tensor");
        }
    }
    if ((rc = check_device())) return rc;
    // the no-allocation variant keeps its workspace in the static scratch:
    // order [N], (checkpoints) chunk offsets [N + 1], the 16-byte check result
    const size_t ws_bytes = cu_seqlens ? 4 * static_cast<size_t>(p.n_seq) +
                                             (hck ? 4 * static_cast<size_t>(p.n_seq + 1) : 0) + 16
                                       : 0;
    if (noalloc && ws_bytes > gdr::kScratchBytes)
        return fail(GDR_ESHAPE,
                    "no-allocation entry point: %lld sequences need %zu bytes of workspace, more than its %zu-byte "
                    "scratch (at most %zu sequences); use gdr_chunk_fwd",
                    (long long)p.n_seq, ws_bytes, gdr::kScratchBytes, (gdr::kScratchBytes - 16) / 4);
    if (p.n_seq == 0 || p.total_tokens == 0) return ok();

    gdr::FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    if ((rc = fwd_defaults(a))) return rc;
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.g = g->data;
    a.beta = beta->data;
    a.cu = cu_seqlens ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
    a.order = nullptr;
    a.h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
    a.o = o->data;
    a.ht = ht ? static_cast<float *>(ht->data) : nullptr;
    a.n_seq = p.n_seq;
    a.seq_len = cu_seqlens ? p.total_tokens : q->shape[1];
    a.total_tokens = p.total_tokens;
    a.hk = p.hk;
    a.hv = p.hv;
    a.d = p.d;
    a.dv = p.dv;
    a.in_bf16 = p.in_dtype == GDR_BF16;
    a.gate_bf16 = p.gate_dtype == GDR_BF16;
    a.scale = scale;
    a.hck = hck ? static_cast<float *>(hck->data) : nullptr;
    a.ck_offs = nullptr;
    a.ck_rows = rows;
    a.ck_every = static_cast<int32_t>(every);

    WsLease lease;
    if (cu_seqlens) {
        void *ws = nullptr;
        if (noalloc) {
            const hipError_t e = gdr::device_buffers(nullptr, &ws);
            if (e != hipSuccess) return fail(GDR_EDEVICE, "scratch of the no-allocation entry point: %s",
                                             hipGetErrorString(e));
        } else if ((rc = lease.acquire(ws_bytes, false, stream, &ws))) {
            return rc;
        }
        int32_t *order = static_cast<int32_t *>(ws);
        int32_t *offs = hck ? order + p.n_seq : nullptr;
        int32_t *check = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(ws) + ws_bytes - 16);
        if ((rc = check_cu_content(a.cu, p.n_seq, p.total_tokens, check, stream))) return rc;
        const int groups = hck ? 0 : order_groups(a);
        const hipError_t e = groups ? gdr::launch_order(a.cu, p.n_seq, groups, order, stream)
                                    : gdr::launch_prepare(a.cu, p.n_seq, offs, nullptr, 0, order, stream,
                                                          static_cast<int32_t>(every));
        if (e != hipSuccess) return launch_error(e, "chunk preparation kernel");
        a.order = order;
        a.ck_offs = offs;
    }
    const hipError_t e = launch_or_fail(gdr::launch_fwd, a, stream);
    const int rr = lease.release();
    if (e != hipSuccess) return launch_error(e, "forward kernel");
    return rr ? rr : ok();
}

// Workspace of a backward call: chunk indices (varlen only), then per (chunk
// row, v-head) the forward state, the state gradient, dU and T^T, each part
// 256-byte aligned.
struct BwdWorkspace {
    size_t ints, hck, dhe, du, tmat, total;
};
BwdWorkspace bwd_workspace(int64_t n_seq, int64_t rows, int64_t hv, int64_t d, bool varlen) {
    auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    const size_t ch = static_cast<size_t>(rows) * static_cast<size_t>(hv);
    const size_t dd = static_cast<size_t>(d);
    BwdWorkspace w;
    size_t o = 0;
    w.ints = o;
    o += al(varlen ? 4 * static_cast<size_t>(2 * n_seq + 1 + 2 * rows + 4) : 0);
    w.hck = o;
    o += al(ch * dd * dd * 2);
    w.dhe = o;
    o += al(ch * dd * dd * 2);
    w.du = o;
    o += al(ch * gdr::kChunk * dd * 2);
    w.tmat = o;
    o += al(ch * gdr::kChunk * gdr::kChunk * 2);
    w.total = o;
    return w;
}

int check_out(const gdr_tensor *t, const char *name, int ndim, int32_t dtype, std::initializer_list<int64_t> shape,
              int64_t *numel) {
    int rc = check_tensor(t, name, ndim, numel, 16);
    if (rc) return rc;
    if (t->dtype != dtype) return fail(GDR_EDTYPE, "%s: dtype must be %s, got %s", name, dtype_name(dtype), dtype_name(t->dtype));
    if (!shape_is(t, shape)) return fail(GDR_ESHAPE, "%s: shape %s does not match the inputs", name, shape_str(t).c_str());
    return GDR_OK;
}

int run_bwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
            const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0, const gdr_tensor *dout,
            const gdr_tensor *dht, const gdr_tensor *dq, const gdr_tensor *dk, const gdr_tensor *dv,
            const gdr_tensor *dg, const gdr_tensor *dbeta, const gdr_tensor *dh0, float scale, hipStream_t stream) {
    gdr_launch_plan p;
    int rc = plan_fwd(q, k, v, g, beta, cu_seqlens, h0, dout, nullptr, scale, &p, "do");
    if (rc) return rc;
    if (p.d != p.dv)
        return fail(GDR_ESHAPE, "gdr_chunk_bwd needs dk == dv (got dk = %d, dv = %d)", p.d, p.dv);
    const int64_t B = q->shape[0], T = q->shape[1], N = p.n_seq, Hk = p.hk, Hv = p.hv, d = p.d;
    int64_t ndht = 0, ndq, ndk, ndv, ndg, ndb, ndh0 = 0;
    if (dht) {
        if ((rc = check_tensor(dht, "dht", 4, &ndht, 4))) return rc;
        if (dht->dtype != GDR_F32) return fail(GDR_EDTYPE, "dht: dtype must be f32");
        if (!shape_is(dht, {N, Hv, d, d}))
            return fail(GDR_ESHAPE, "dht: shape %s must be [N, Hv, dk, dv]", shape_str(dht).c_str());
    }
    if ((rc = check_out(dq, "dq", 4, q->dtype, {B, T, Hk, d}, &ndq))) return rc;
    if ((rc = check_out(dk, "dk", 4, q->dtype, {B, T, Hk, d}, &ndk))) return rc;
    if ((rc = check_out(dv, "dv", 4, q->dtype, {B, T, Hv, d}, &ndv))) return rc;
    if ((rc = check_out(dg, "dg", 3, GDR_F32, {B, T, Hv}, &ndg))) return rc;
    if ((rc = check_out(dbeta, "dbeta", 3, GDR_F32, {B, T, Hv}, &ndb))) return rc;
    if (dh0 && (rc = check_out(dh0, "dh0", 4, GDR_F32, {N, Hv, d, d}, &ndh0))) return rc;

    auto numel = [](const gdr_tensor *t) {
        int64_t n = 1;
        for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
        return n;
    };
    const gdr_tensor *ins[] = {q, k, v, g, beta, cu_seqlens, h0, dout, dht};
    const Span outs[] = {span_of(dq, ndq), span_of(dk, ndk), span_of(dv, ndv), span_of(dg, ndg),
                         span_of(dbeta, ndb), span_of(dh0, ndh0)};
    for (const gdr_tensor *t : ins) {
        if (!t) continue;
        const Span si = span_of(t, numel(t));
        for (const Span &so : outs)
            if (overlap(so, si)) return fail(GDR_EALIAS, "a gradient output overlaps an input");
    }
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return fail(GDR_EALIAS, "gradient outputs overlap");
    if ((rc = check_device())) return rc;
    if (N == 0 || p.total_tokens == 0) return ok();

    const bool varlen = cu_seqlens != nullptr;
    const int64_t rows = varlen ? p.nt_max : B * ((T + gdr::kChunk - 1) / gdr::kChunk);
    const BwdWorkspace wl = bwd_workspace(N, rows, Hv, d, varlen);
    gdr::FwdArgs fa;
    std::memset(&fa, 0, sizeof(fa));
    if ((rc = fwd_defaults(fa))) return rc;
    WsLease lease;
    void *ws = nullptr;
    if ((rc = lease.acquire(wl.total, true, stream, &ws))) return rc;
    unsigned char *base = static_cast<unsigned char *>(ws);
    int32_t *offs = nullptr, *map = nullptr, *order = nullptr;
    const int32_t *cu = varlen ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
    hipError_t e = hipSuccess;
    if (varlen) {
        offs = reinterpret_cast<int32_t *>(base + wl.ints);
        map = offs + N + 1;
        order = map + 2 * rows;
        if ((rc = check_cu_content(cu, N, p.total_tokens, order + N, stream))) return rc;
        e = gdr::launch_prepare(cu, N, offs, map, rows, order, stream);
    }
    uint16_t *hck = reinterpret_cast<uint16_t *>(base + wl.hck);
    if (e == hipSuccess) {
        // forward recompute: the state after every chunk (no o, no ht)
        fa.q = q->data;
        fa.k = k->data;
        fa.v = v->data;
        fa.g = g->data;
        fa.beta = beta->data;
        fa.cu = cu;
        fa.order = order;
        fa.h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
        fa.o = nullptr;
        fa.ht = nullptr;
        fa.n_seq = N;
        fa.seq_len = varlen ? p.total_tokens : T;
        fa.total_tokens = p.total_tokens;
        fa.hk = p.hk;
        fa.hv = p.hv;
        fa.d = p.d;
        fa.dv = p.dv;
        fa.in_bf16 = p.in_dtype == GDR_BF16;
        fa.gate_bf16 = p.gate_dtype == GDR_BF16;
        fa.scale = scale;
        fa.hck16 = hck;
        fa.ck_offs = offs;
        fa.ck_rows = rows;
        e = gdr::launch_fwd(fa, stream);
    }
    if (e == hipSuccess) {
        gdr::BwdArgs ba;
        std::memset(&ba, 0, sizeof(ba));
        ba.q = q->data;
        ba.k = k->data;
        ba.v = v->data;
        ba.g = g->data;
        ba.beta = beta->data;
        ba.dout = dout->data;
        ba.cu = cu;
        ba.map = map;
        ba.offs = offs;
        ba.order = order;
        ba.h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
        ba.dht = dht ? static_cast<const float *>(dht->data) : nullptr;
        ba.hck = hck;
        ba.tmat = reinterpret_cast<uint16_t *>(base + wl.tmat);
        ba.du = reinterpret_cast<uint16_t *>(base + wl.du);
        ba.dhe = reinterpret_cast<uint16_t *>(base + wl.dhe);
        ba.dq = dq->data;
        ba.dk = dk->data;
        ba.dv = dv->data;
        ba.dg = static_cast<float *>(dg->data);
        ba.dbeta = static_cast<float *>(dbeta->data);
        ba.dh0 = dh0 ? static_cast<float *>(dh0->data) : nullptr;
        ba.n_seq = N;
        ba.seq_len = varlen ? p.total_tokens : T;
        ba.total_tokens = p.total_tokens;
        ba.rows = rows;
        ba.hk = p.hk;
        ba.hv = p.hv;
        ba.d = p.d;
        ba.in_bf16 = p.in_dtype == GDR_BF16;
        ba.gate_bf16 = p.gate_dtype == GDR_BF16;
        ba.scale = scale;
        e = forced_failure() ? hipErrorLaunchFailure : gdr::launch_bwd(ba, stream);
    }
    const int rr = lease.release();
    if (e != hipSuccess) return launch_error(e, "backward kernels");
    return rr ? rr : ok();
}

// The per-channel-gate forward: g is [B, T, Hv, dk]; everything else is
// validated as for gdr_chunk_fwd (with beta standing in for the scalar g).
int run_kda(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
            const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0, const gdr_tensor *o,
            const gdr_tensor *ht, float scale, hipStream_t stream) {
    int64_t ng;
    int rc;
    if ((rc = check_tensor(g, "g", 4, &ng, 4))) return rc;
    gdr_launch_plan p;
    if ((rc = plan_fwd(q, k, v, beta, beta, cu_seqlens, h0, o, ht, scale, &p))) return rc;
    if (p.d != p.dv)
        return fail(GDR_ESHAPE, "gdr_chunk_kda_fwd needs dk == dv (got dk = %d, dv = %d)", p.d, p.dv);
    if (g->dtype != beta->dtype) return fail(GDR_EDTYPE, "g and beta must share one dtype");
    const int64_t B = q->shape[0], T = q->shape[1];
    if (!shape_is(g, {B, T, p.hv, p.d}))
        return fail(GDR_ESHAPE, "g: shape %s must be [B, T, Hv, dk]", shape_str(g).c_str());
    int64_t no = 1, nht = 1;
    for (int i = 0; i < 4; ++i) no *= o->shape[i];
    if (ht)
        for (int i = 0; i < 4; ++i) nht *= ht->shape[i];
    const Span sg = span_of(g, ng);
    if (overlap(span_of(o, no), sg)) return fail(GDR_EALIAS, "o overlaps an input");
    if (ht && overlap(span_of(ht, nht), sg)) return fail(GDR_EALIAS, "ht overlaps an input");
    if ((rc = check_device())) return rc;
    if (p.n_seq == 0 || p.total_tokens == 0) return ok();

    gdr::FwdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.g = g->data;
    a.beta = beta->data;
    a.cu = cu_seqlens ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
    a.h0 = h0 ? static_cast<const float *>(h0->data) : nullptr;
    a.o = o->data;
    a.ht = ht ? static_cast<float *>(ht->data) : nullptr;
    a.n_seq = p.n_seq;
    a.seq_len = cu_seqlens ? p.total_tokens : T;
    a.total_tokens = p.total_tokens;
    a.hk = p.hk;
    a.hv = p.hv;
    a.d = p.d;
    a.dv = p.dv;
    a.in_bf16 = p.in_dtype == GDR_BF16;
    a.gate_bf16 = p.gate_dtype == GDR_BF16;
    a.scale = scale;
    if ((rc = fwd_defaults(a))) return rc;
    WsLease lease;
    hipError_t e = hipSuccess;
    if (cu_seqlens) {   // the packed dispatch order where it applies, else longest sequences first
        void *ws = nullptr;
        if ((rc = lease.acquire(static_cast<size_t>(4 * p.n_seq + 16), false, stream, &ws))) return rc;
        int32_t *order = static_cast<int32_t *>(ws);
        if ((rc = check_cu_content(a.cu, p.n_seq, p.total_tokens, order + p.n_seq, stream))) return rc;
        a.order = order;
        const int groups = order_groups(a, true);
        e = groups ? gdr::launch_order(a.cu, p.n_seq, groups, order, stream)
                   : gdr::launch_prepare(a.cu, p.n_seq, nullptr, nullptr, 0, order, stream);
    }
    if (e == hipSuccess) e = launch_or_fail(gdr::launch_kda_fwd, a, stream);
    const int rr = lease.release();
    if (e != hipSuccess) return launch_error(e, "per-channel-gate forward kernel");
    return rr ? rr : ok();
}

}  // namespace

extern "C" {

int gdr_plan(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
             const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
             const gdr_tensor *o, const gdr_tensor *ht, float scale, gdr_launch_plan *plan) {
    if (!plan) return fail(GDR_EINVAL, "plan is NULL");
    const int rc = plan_fwd(q, k, v, g, beta, cu_seqlens, h0, o, ht, scale, plan);
    return rc ? rc : ok();
}

int gdr_chunk_fwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                  const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                  const gdr_tensor *o, const gdr_tensor *ht, float scale, hipStream_t stream) {
    return run_fwd(q, k, v, g, beta, cu_seqlens, h0, o, ht, nullptr, scale, stream);
}

int gdr_chunk_fwd_checkpoints(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                              const gdr_tensor *g, const gdr_tensor *beta, const gdr_tensor *cu_seqlens,
                              const gdr_tensor *h0, const gdr_tensor *o, const gdr_tensor *ht,
                              const gdr_tensor *h_chunks, float scale, hipStream_t stream) {
    if (!h_chunks) return fail(GDR_EINVAL, "h_chunks: descriptor is NULL");
    return run_fwd(q, k, v, g, beta, cu_seqlens, h0, o, ht, h_chunks, scale, stream);
}

int gdr_chunk_fwd_checkpoints_n(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                                const gdr_tensor *g, const gdr_tensor *beta, const gdr_tensor *cu_seqlens,
                                const gdr_tensor *h0, const gdr_tensor *o, const gdr_tensor *ht,
                                const gdr_tensor *h_ckpt, int64_t every_n, float scale, hipStream_t stream) {
    if (!h_ckpt) return fail(GDR_EINVAL, "h_ckpt: descriptor is NULL");
    return run_fwd(q, k, v, g, beta, cu_seqlens, h0, o, ht, h_ckpt, scale, stream, false, every_n);
}

int gdr_chunk_bwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                  const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                  const gdr_tensor *dout, const gdr_tensor *dht, const gdr_tensor *dq, const gdr_tensor *dk,
                  const gdr_tensor *dv, const gdr_tensor *dg, const gdr_tensor *dbeta, const gdr_tensor *dh0,
                  float scale, hipStream_t stream) {
    return run_bwd(q, k, v, g, beta, cu_seqlens, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0, scale, stream);
}

int gdr_chunk_kda_fwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                      const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                      const gdr_tensor *o, const gdr_tensor *ht, float scale, hipStream_t stream) {
    return run_kda(q, k, v, g, beta, cu_seqlens, h0, o, ht, scale, stream);
}

int gdr_decode_step(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                    const gdr_tensor *beta, const gdr_tensor *h, const gdr_tensor *o, float scale,
                    hipStream_t stream) {
    int64_t nq, nk, nv, ng, nb, nh, no;
    int rc;
    if ((rc = check_tensor(q, "q", 3, &nq, 8))) return rc;
    if ((rc = check_tensor(k, "k", 3, &nk, 8))) return rc;
    if ((rc = check_tensor(v, "v", 3, &nv, 8))) return rc;
    if ((rc = check_tensor(g, "g", 2, &ng, 4))) return rc;
    if ((rc = check_tensor(beta, "beta", 2, &nb, 4))) return rc;
    if ((rc = check_tensor(h, "h", 4, &nh, 16))) return rc;
    if ((rc = check_tensor(o, "o", 3, &no, 16))) return rc;
    if (q->dtype != GDR_BF16 && q->dtype != GDR_F32)
        return fail(GDR_EDTYPE, "q: dtype must be bf16 or f32, got %s", dtype_name(q->dtype));
    if (k->dtype != q->dtype || v->dtype != q->dtype || o->dtype != q->dtype)
        return fail(GDR_EDTYPE, "q, k, v and o must share one dtype (q is %s)", dtype_name(q->dtype));
    if (g->dtype != GDR_BF16 && g->dtype != GDR_F32)
        return fail(GDR_EDTYPE, "g: dtype must be bf16 or f32, got %s", dtype_name(g->dtype));
    if (beta->dtype != g->dtype) return fail(GDR_EDTYPE, "beta must have the dtype of g");
    if (h->dtype != GDR_F32) return fail(GDR_EDTYPE, "h: dtype must be f32");
    const int64_t B = q->shape[0], Hk = q->shape[1], d = q->shape[2];
    const int64_t Hv = v->shape[1], dv = v->shape[2];
    if (!shape_is(k, {B, Hk, d}))
        return fail(GDR_ESHAPE, "k: shape %s must equal q's %s", shape_str(k).c_str(), shape_str(q).c_str());
    if (v->shape[0] != B)
        return fail(GDR_ESHAPE, "v: shape %s must be [B, Hv, dv] with q's B", shape_str(v).c_str());
    if (!shape_is(o, {B, Hv, dv}))
        return fail(GDR_ESHAPE, "o: shape %s must equal v's %s", shape_str(o).c_str(), shape_str(v).c_str());
    if (!shape_is(g, {B, Hv}) || !shape_is(beta, {B, Hv}))
        return fail(GDR_ESHAPE, "g and beta must be [B, Hv] = [%lld, %lld]", (long long)B, (long long)Hv);
    if (!shape_is(h, {B, Hv, d, dv}))
        return fail(GDR_ESHAPE, "h: shape %s must be [B, Hv, dk, dv] = [%lld, %lld, %lld, %lld]",
                    shape_str(h).c_str(), (long long)B, (long long)Hv, (long long)d, (long long)dv);
    if (d != 64 && d != 128) return fail(GDR_ESHAPE, "dk must be 64 or 128, got %lld", (long long)d);
    if (dv != 64 && dv != 128) return fail(GDR_ESHAPE, "dv must be 64 or 128, got %lld", (long long)dv);
    if (Hk < 1 || Hv < 1) return fail(GDR_ESHAPE, "head counts must be positive");
    if (Hv % Hk != 0)
        return fail(GDR_ESHAPE, "Hv (%lld) must be a multiple of Hk (%lld)", (long long)Hv, (long long)Hk);
    if (B * Hv > 0x7FFFFFFFLL) return fail(GDR_ESHAPE, "B * Hv exceeds the launch grid limit");
    if (!std::isfinite(scale)) return fail(GDR_EINVAL, "scale must be finite");
    const Span so = span_of(o, no), sh = span_of(h, nh);
    const Span ins[] = {span_of(q, nq), span_of(k, nk), span_of(v, nv), span_of(g, ng), span_of(beta, nb)};
    for (const Span &x : ins) {
        if (overlap(so, x)) return fail(GDR_EALIAS, "o overlaps an input");
        if (overlap(sh, x)) return fail(GDR_EALIAS, "h overlaps an input");
    }
    if (overlap(so, sh)) return fail(GDR_EALIAS, "o and h overlap");
    if ((rc = check_device())) return rc;
    if (B == 0) return ok();
    gdr::DecodeArgs a;
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.g = g->data;
    a.beta = beta->data;
    a.h = static_cast<float *>(h->data);
    a.o = o->data;
    a.batch = B;
    a.hk = static_cast<int32_t>(Hk);
    a.hv = static_cast<int32_t>(Hv);
    a.d = static_cast<int32_t>(d);
    a.dv = static_cast<int32_t>(dv);
    a.in_bf16 = q->dtype == GDR_BF16;
    a.gate_bf16 = g->dtype == GDR_BF16;
    a.scale = scale;
    const hipError_t e = forced_failure() ? hipErrorLaunchFailure : gdr::launch_decode(a, stream);
    if (e != hipSuccess) return launch_error(e, "decode kernel");
    return ok();
}

int gdr_dispatch_order(const gdr_tensor *cu_seqlens, int32_t groups, const gdr_tensor *order,
                       hipStream_t stream) {
    int64_t ncu, nord;
    int rc;
    if ((rc = check_tensor(cu_seqlens, "cu_seqlens", 1, &ncu, 4))) return rc;
    if ((rc = check_tensor(order, "order", 1, &nord, 4))) return rc;
    if (cu_seqlens->dtype != GDR_I32 || order->dtype != GDR_I32) return fail(GDR_EDTYPE, "cu_seqlens and order must be i32");
    const int64_t N = ncu - 1;
    if (N < 1 || N > 64) return fail(GDR_ESHAPE, "dispatch order needs 1 <= N <= 64 sequences, got %lld", (long long)N);
    if (nord != N) return fail(GDR_ESHAPE, "order must have N = %lld entries", (long long)N);
    if (groups < 1 || groups > 16) return fail(GDR_EINVAL, "groups must be in [1, 16], got %d", groups);
    if (overlap(span_of(cu_seqlens, ncu), span_of(order, nord))) return fail(GDR_EALIAS, "order overlaps cu_seqlens");
    if ((rc = check_device())) return rc;
    const hipError_t e = gdr::launch_order(static_cast<const int32_t *>(cu_seqlens->data), N, groups,
                                           static_cast<int32_t *>(order->data), stream);
    if (e != hipSuccess) return launch_error(e, "dispatch order kernel");
    return ok();
}

int gdr_prepare_chunks(const gdr_tensor *cu_seqlens, const gdr_tensor *chunk_offsets,
                       const gdr_tensor *chunk_map, const gdr_tensor *seq_order, hipStream_t stream) {
    int64_t ncu, noff, nmap = 0, nord = 0;
    int rc;
    if ((rc = check_tensor(cu_seqlens, "cu_seqlens", 1, &ncu, 4))) return rc;
    if ((rc = check_tensor(chunk_offsets, "chunk_offsets", 1, &noff, 4))) return rc;
    if (chunk_map && (rc = check_tensor(chunk_map, "chunk_map", 2, &nmap, 4))) return rc;
    if (seq_order && (rc = check_tensor(seq_order, "seq_order", 1, &nord, 4))) return rc;
    if (cu_seqlens->dtype != GDR_I32 || chunk_offsets->dtype != GDR_I32 ||
        (chunk_map && chunk_map->dtype != GDR_I32) || (seq_order && seq_order->dtype != GDR_I32))
        return fail(GDR_EDTYPE, "chunk preparation tensors must be i32");
    if (ncu < 1) return fail(GDR_ESHAPE, "cu_seqlens must hold at least one offset");
    const int64_t N = ncu - 1;
    if (noff != N + 1) return fail(GDR_ESHAPE, "chunk_offsets must have N + 1 = %lld entries", (long long)(N + 1));
    if (chunk_map && chunk_map->shape[1] != 2) return fail(GDR_ESHAPE, "chunk_map must be [nt_max, 2]");
    if (seq_order && nord != N) return fail(GDR_ESHAPE, "seq_order must have N = %lld entries", (long long)N);
    const Span in = span_of(cu_seqlens, ncu);
    const Span outs[] = {span_of(chunk_offsets, noff), span_of(chunk_map, nmap), span_of(seq_order, nord)};
    for (int i = 0; i < 3; ++i) {
        if (overlap(in, outs[i])) return fail(GDR_EALIAS, "an output overlaps cu_seqlens");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(GDR_EALIAS, "outputs overlap");
    }
    if ((rc = check_device())) return rc;
    const hipError_t e = gdr::launch_prepare(
        static_cast<const int32_t *>(cu_seqlens->data), N, static_cast<int32_t *>(chunk_offsets->data),
        chunk_map ? static_cast<int32_t *>(chunk_map->data) : nullptr, chunk_map ? chunk_map->shape[0] : 0,
        seq_order ? static_cast<int32_t *>(seq_order->data) : nullptr, stream);
    if (e != hipSuccess) return launch_error(e, "chunk preparation kernel");
    return ok();
}

int gdr_chunk_local_cumsum(const gdr_tensor *g, const gdr_tensor *cu_seqlens, const gdr_tensor *G,
                           hipStream_t stream) {
    int64_t ng, ncu = 0, nG;
    int rc;
    if ((rc = check_tensor(g, "g", 3, &ng, 4))) return rc;
    if (cu_seqlens && (rc = check_tensor(cu_seqlens, "cu_seqlens", 1, &ncu, 4))) return rc;
    if ((rc = check_tensor(G, "G", 3, &nG, 4))) return rc;
    if (g->dtype != GDR_BF16 && g->dtype != GDR_F32) return fail(GDR_EDTYPE, "g: dtype must be bf16 or f32");
    if (G->dtype != GDR_F32) return fail(GDR_EDTYPE, "G: dtype must be f32");
    if (cu_seqlens && cu_seqlens->dtype != GDR_I32) return fail(GDR_EDTYPE, "cu_seqlens: dtype must be i32");
    const int64_t B = g->shape[0], T = g->shape[1], H = g->shape[2];
    if (!shape_is(G, {B, T, H})) return fail(GDR_ESHAPE, "G must have the shape of g");
    if (H > 0x7FFFFFFF) return fail(GDR_ESHAPE, "too many heads");
    if (cu_seqlens && B != 1) return fail(GDR_ESHAPE, "cu_seqlens requires B == 1");
    if (cu_seqlens && ncu < 1) return fail(GDR_ESHAPE, "cu_seqlens must hold at least one offset");
    if (overlap(span_of(G, nG), span_of(g, ng)) || overlap(span_of(G, nG), span_of(cu_seqlens, ncu)))
        return fail(GDR_EALIAS, "G overlaps an input");
    if (B * T > 0x7FFFFFFFLL) return fail(GDR_ESHAPE, "B * T exceeds 2^31 - 1 tokens");
    if ((rc = check_device())) return rc;
    if (B * T == 0 || H == 0) return ok();
    const int gate_bf16 = g->dtype == GDR_BF16;
    if (!cu_seqlens) {
        const hipError_t e = forced_failure() ? hipErrorLaunchFailure
                                              : gdr::launch_cumsum(g->data, gate_bf16, nullptr, nullptr, 0, B, T, B * T,
                                                                   static_cast<int32_t>(H),
                                                                   static_cast<float *>(G->data), stream);
        if (e != hipSuccess) return launch_error(e, "cumsum kernel");
        return ok();
    }
    const int64_t N = ncu - 1;
    if (N == 0) return ok();
    const int64_t nt_max = (T + gdr::kChunk - 1) / gdr::kChunk + N;
    if (nt_max > 0x7FFFFFFFLL) return fail(GDR_ESHAPE, "too many chunks");
    void *ws = nullptr;
    const size_t bytes = static_cast<size_t>(nt_max) * 8 + 16;
    WsLease lease;
    if ((rc = lease.acquire(bytes, false, stream, &ws))) return rc;
    hipError_t e;
    int32_t *map = static_cast<int32_t *>(ws);
    const int32_t *cu = static_cast<const int32_t *>(cu_seqlens->data);
    if ((rc = check_cu_content(cu, N, T, map + 2 * nt_max, stream))) return rc;
    e = gdr::launch_prepare(cu, N, nullptr, map, nt_max, nullptr, stream);
    if (e == hipSuccess)
        e = forced_failure() ? hipErrorLaunchFailure
                             : gdr::launch_cumsum(g->data, gate_bf16, cu, map, nt_max, 1, T, T, static_cast<int32_t>(H),
                                                  static_cast<float *>(G->data), stream);
    const int rr = lease.release();
    if (e != hipSuccess) return launch_error(e, "chunk preparation / cumsum kernels");
    return rr ? rr : ok();
}

int gdr_chunk_fwd_noalloc(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                          const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                          const gdr_tensor *o, const gdr_tensor *ht, float scale, hipStream_t stream) {
    return run_fwd(q, k, v, g, beta, cu_seqlens, h0, o, ht, nullptr, scale, stream, true);
}

int gdr_debug_set(int option, int64_t value) {
    switch (option) {
    case GDR_DEBUG_CHECK_CU:
        g_check_cu.store(value != 0 ? 1 : 0);
        return ok();
    case GDR_DEBUG_FAIL_LAUNCHES:
        if (value < 0) return fail(GDR_EINVAL, "GDR_DEBUG_FAIL_LAUNCHES: count must be >= 0, got %lld", (long long)value);
        g_fail_launches.store(value);
        return ok();
    case GDR_DEBUG_SPIN_LIMIT:
        if (value > 0x7FFFFFFF) return fail(GDR_EINVAL, "GDR_DEBUG_SPIN_LIMIT: at most 2^31 - 1 polls");
        g_spin_max.store(value < 0 ? gdr::kSpinDefault : static_cast<int32_t>(value));
        return ok();
    default:
        return fail(GDR_EINVAL, "gdr_debug_set: unknown option %d", option);
    }
}

int gdr_device_status(uint32_t *bits, int clear) {
    if (!bits) return fail(GDR_EINVAL, "gdr_device_status: bits is NULL");
    int rc;
    if ((rc = check_device())) return rc;
    uint32_t *st = nullptr;
    hipError_t e = gdr::device_buffers(&st, nullptr);
    if (e != hipSuccess) return fail(GDR_EDEVICE, "device status word: %s", hipGetErrorString(e));
    if ((e = hipDeviceSynchronize()) != hipSuccess) return launch_error(e, "gdr_device_status: synchronise");
    if ((e = hipMemcpy(bits, st, sizeof(uint32_t), hipMemcpyDeviceToHost)) != hipSuccess)
        return launch_error(e, "gdr_device_status: read");
    if (clear) {
        const uint32_t zero = 0;
        if ((e = hipMemcpy(st, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess)
            return launch_error(e, "gdr_device_status: clear");
    }
    return ok();
}

int gdr_free_workspaces(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(GDR_EDEVICE, "no current device");
    WsDevice &D = g_ws[dev];
    std::lock_guard<std::mutex> g(D.mu);
    std::unique_lock<std::mutex> locks[kRing];
    for (int i = 0; i < kRing; ++i) locks[i] = std::unique_lock<std::mutex>(D.ring[i].mu);
    std::lock_guard<std::mutex> gb(D.big.mu);
    for (WsSlot *s : {&D.ring[0], &D.ring[1], &D.ring[2], &D.ring[3], &D.ring[4], &D.ring[5], &D.ring[6],
                      &D.ring[7], &D.big}) {
        if (s->used) (void)hipEventSynchronize(s->ev);
        s->used = false;
        if (s->ev) (void)hipEventDestroy(s->ev);
        s->ev = nullptr;
    }
    static_assert(kRing == 8, "the list above names every ring slot");
    hipError_t e = hipSuccess;
    if (D.block) e = hipFree(D.block);
    if (D.big_ptr) {
        const hipError_t e2 = hipFree(D.big_ptr);
        if (e == hipSuccess) e = e2;
    }
    D.block = nullptr;
    D.cap = 0;
    D.big_ptr = nullptr;
    D.big_cap = 0;
    if (e != hipSuccess) return launch_error(e, "gdr_free_workspaces");
    return ok();
}

const char *gdr_last_error(void) { return g_last_error.c_str(); }

int gdr_version(void) { return 10300; }

int gdr_selftest_mfma(const uint16_t *a, const uint16_t *b, float *c, hipStream_t stream) {
    if (!a || !b || !c) return fail(GDR_EINVAL, "selftest: NULL pointer");
    int rc;
    if ((rc = check_device())) return rc;
    const hipError_t e = gdr::launch_selftest_mfma(a, b, c, stream);
    if (e != hipSuccess) return launch_error(e, "selftest kernel");
    return ok();
}

}  // extern "C"
