// rwkvwkv_abi.hip -- the C ABI of librwkvwkv: argument validation, algorithm choice,
// workspace management and launch.  Every check runs on the host before anything is
// enqueued, so an error return leaves all outputs untouched.

#include "rwkvwkv.h"
#include "wkv_internal.h"

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

using namespace rwkvwkv;

namespace {

thread_local char g_err[512];

rwkv_status fail(rwkv_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

rwkv_status ok() {
    g_err[0] = 0;
    return RWKV_OK;
}

rwkv_status hip_fail(hipError_t e, const char *where) {
    return fail(RWKV_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Library-cached chunked-scan workspace, one per (device, stream), grown on demand.  Calls on
// one stream run in order, so they may share one; calls on different streams may run at once
// and must not share the look-back words.
struct CachedWorkspace {
    int dev;
    hipStream_t stream;
    void *ptr;
    size_t bytes;
};
std::mutex g_ws_mu;
std::vector<CachedWorkspace> g_ws;
std::atomic<uint32_t> g_epoch{0};

// Launch stamp in [1, 2^30 - 1]; a zero-filled workspace never matches it.
uint32_t next_epoch() { return (g_epoch.fetch_add(1, std::memory_order_relaxed) % ((1u << 30) - 1u)) + 1u; }

// The cached workspace of (current device, stream), or null if none was allocated yet.
CachedWorkspace *find_cached(int dev, hipStream_t stream) {
    for (CachedWorkspace &w : g_ws)
        if (w.dev == dev && w.stream == stream) return &w;
    return nullptr;
}

rwkv_status cached_workspace(size_t need, hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_ws_mu);
    CachedWorkspace *w = find_cached(dev, stream);
    if (!w) {
        g_ws.push_back(CachedWorkspace{dev, stream, nullptr, 0});
        w = &g_ws.back();
    }
    if (w->bytes < need) {
        if (w->ptr) {
            // the old buffer may still be in use by work enqueued on the stream
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            (void)hipFree(w->ptr);
            w->ptr = nullptr;
            w->bytes = 0;
        }
        size_t nb = need < (1u << 20) ? (1u << 20) : need;
        void *p = nullptr;
        e = hipMalloc(&p, nb);
        if (e != hipSuccess) return fail(RWKV_ERR_NOMEM, "workspace of %zu bytes: %s", nb, hipGetErrorString(e));
        e = hipMemsetAsync(p, 0, nb, stream);
        if (e != hipSuccess) {
            (void)hipFree(p);
            return hip_fail(e, "hipMemsetAsync(workspace)");
        }
        w->ptr = p;
        w->bytes = nb;
    }
    *out = w->ptr;
    return RWKV_OK;
}

// Scratch of rwkv4_timemix_fused_noalloc, for callers that cannot allocate: the two-pass scan's
// tile aggregates (16 bytes per channel and tile, 16 MiB in all).  Each GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name only stands in for
// the symbol: its device address on each GPU comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is ever handed to a kernel.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

rwkv_status static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(RWKV_ERR_ARG, "device %d: at most %d devices", dev,
                                                          kMaxScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(RWKV_ERR_HIP, "hipGetSymbolAddress(scratch) returned no address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RWKV_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void *p, size_t pn, const void *q, size_t qn) {
    if (!p || !q || !pn || !qn) return false;
    const char *a = (const char *)p, *b = (const char *)q;
    return a < b + qn && b < a + pn;
}

const int64_t kMaxElems = (int64_t)1 << 46;

rwkv_status check_dtype(int32_t d, const char *what) {
    if (d != RWKV_F32 && d != RWKV_F16 && d != RWKV_BF16)
        return fail(RWKV_ERR_DTYPE, "%s: unknown dtype %d", what, (int)d);
    return RWKV_OK;
}

size_t esize(int32_t d) { return d == RWKV_F32 ? 4 : 2; }

struct Resolved {
    int32_t in_dtype = RWKV_F32, out_dtype = RWKV_F32;
    const void *r = nullptr;
    int32_t chunk_len = 0, algo = RWKV_ALGO_AUTO;
    void *workspace = nullptr;
    size_t workspace_bytes = 0;
    int32_t publish = RWKV_PUBLISH_AUTO;
    bool static_scratch = false;  // rwkv4_timemix_fused_noalloc: the two-pass scan on the static scratch
};

rwkv_status resolve_opts(const rwkv4_opts *o, Resolved *r) {
    if (!o) return RWKV_OK;
    const bool has_publish = o->size == sizeof(rwkv4_opts);
    if (!has_publish && o->size != offsetof(rwkv4_opts, publish))
        return fail(RWKV_ERR_ARG, "opts->size is %u, expected sizeof(rwkv4_opts) = %zu", o->size,
                    sizeof(rwkv4_opts));
    rwkv_status s;
    if ((s = check_dtype(o->in_dtype, "opts->in_dtype")) != RWKV_OK) return s;
    if ((s = check_dtype(o->out_dtype, "opts->out_dtype")) != RWKV_OK) return s;
    if (o->algo < RWKV_ALGO_AUTO || o->algo > RWKV_ALGO_TWO_PASS)
        return fail(RWKV_ERR_ARG, "opts->algo %d is not a rwkv_algo", (int)o->algo);
    if (o->chunk_len != 0) {
        const int c = o->chunk_len;
        if (c < kMinChunk || c > kMaxChunk || (c & (c - 1)) != 0)
            return fail(RWKV_ERR_ARG, "opts->chunk_len %d: must be 0 or a power of two in [%d, %d]", c,
                        kMinChunk, kMaxChunk);
    }
    if (has_publish && (o->publish < RWKV_PUBLISH_AUTO || o->publish > RWKV_PUBLISH_WRITE_THROUGH))
        return fail(RWKV_ERR_ARG, "opts->publish %d is not a rwkv_publish", (int)o->publish);
    if (o->workspace && !aligned(o->workspace, 256))
        return fail(RWKV_ERR_ALIGN, "opts->workspace must be 256-byte aligned");
    r->in_dtype = o->in_dtype;
    r->out_dtype = o->out_dtype;
    r->r = o->r;
    r->chunk_len = o->chunk_len;
    r->algo = o->algo;
    r->workspace = o->workspace;
    r->workspace_bytes = o->workspace_bytes;
    r->publish = has_publish ? o->publish : RWKV_PUBLISH_AUTO;
    return RWKV_OK;
}

// Shared tail of the forward and time-mix entry points: validation of the common
// tensors, algorithm choice, workspace, launch.
rwkv_status run_forward(ForwardArgs &a, const Resolved &o, hipStream_t stream) {
    const int64_t B = a.B, T = a.T, C = a.C;
    if (B < 1 || C < 1 || T < 0) return fail(RWKV_ERR_ARG, "sizes must satisfy B >= 1, C >= 1, T >= 0 (got %lld, %lld, %lld)",
                                              (long long)B, (long long)T, (long long)C);
    if (B > kMaxElems / C || (T > 0 && B * C > kMaxElems / T))
        return fail(RWKV_ERR_ARG, "B*T*C too large");
    if (!a.w || !a.u) return fail(RWKV_ERR_ARG, "w and u are required");
    if (T > 0 && (!a.k || !a.v || !a.y)) return fail(RWKV_ERR_ARG, "k, v and y are required when T > 0");
    const size_t ei = esize(o.in_dtype), eo = esize(o.out_dtype);
    const void *ins[] = {a.k, a.v, a.r, a.x, a.x_prev, a.xk_out, a.xv_out, a.x_last};
    for (const void *p : ins)
        if (p && !aligned(p, ei)) return fail(RWKV_ERR_ALIGN, "activation pointer %p not aligned to %zu bytes", p, ei);
    if (a.y && !aligned(a.y, eo)) return fail(RWKV_ERR_ALIGN, "y not aligned to %zu bytes", eo);
    const float *fl[] = {a.w, a.u, a.mix_k, a.mix_v, a.mix_r, a.state_in, a.state_out};
    for (const float *p : fl)
        if (p && !aligned(p, 4)) return fail(RWKV_ERR_ALIGN, "fp32 pointer %p not 4-byte aligned", (const void *)p);
    const size_t sbytes = (size_t)(3 * B * C) * 4;
    if (a.state_out && a.state_in != a.state_out && overlap(a.state_in, sbytes, a.state_out, sbytes))
        return fail(RWKV_ERR_ARG, "state_out overlaps state_in without being equal to it");
    const size_t abytes_in = (size_t)(B * T * C) * ei, abytes_out = (size_t)(B * T * C) * eo;
    const void *rd[] = {a.k, a.v, a.r, a.x};
    for (const void *p : rd)
        if (overlap(a.y, abytes_out, p, abytes_in)) return fail(RWKV_ERR_ARG, "y overlaps an input");
    if (a.state_out && (overlap(a.state_out, sbytes, a.y, abytes_out)))
        return fail(RWKV_ERR_ARG, "state_out overlaps y");

    a.in_dt = o.in_dtype;
    a.out_dt = o.out_dtype;
    a.publish = o.publish;
    bool vec = (C % 4) == 0;
    for (const void *p : ins)
        if (p && !aligned(p, 4 * ei)) vec = false;
    if (a.y && !aligned(a.y, 4 * eo)) vec = false;
    a.vec = vec ? 1 : 0;
    bool vec16 = (C % (int64_t)(16 / ei)) == 0;
    for (const void *p : {a.k, a.v, a.r, a.x})
        if (p && !aligned(p, 16)) vec16 = false;
    a.vec16 = vec16 ? 1 : 0;
    a.vec16y = (a.y && aligned(a.y, 16) && (C % (int64_t)(16 / eo)) == 0) ? 1 : 0;
    a.vecs = ((C % 4) == 0 && (!a.state_in || aligned(a.state_in, 16)) &&
              (!a.state_out || aligned(a.state_out, 16))) ? 1 : 0;
    bool vecp = (C % 4) == 0;
    for (const float *p : {a.w, a.u, a.mix_k, a.mix_v, a.mix_r})
        if (p && !aligned(p, 16)) vecp = false;
    a.vecp = vecp ? 1 : 0;

    hipError_t e;
    if (T == 0) {
        e = launch_passthrough(a, stream);
        if (e != hipSuccess) return hip_fail(e, "launch (T = 0 state copy)");
        return ok();
    }
    const bool seq = o.algo == RWKV_ALGO_SEQUENTIAL || (o.algo == RWKV_ALGO_AUTO && auto_sequential(B, T, C));
    if (seq) {
        e = launch_sequential(a, stream);
        if (e != hipSuccess) return hip_fail(e, "launch (sequential)");
        return ok();
    }
    const int chunk = o.chunk_len ? o.chunk_len : auto_chunk_len(B, T, C, ei == 2);
    const int tmax = tile_max_len(ei == 2, a.mode != MODE_PLAIN);
    const int64_t nTT = (T + chunk - 1) / chunk;
    bool two_pass = o.algo == RWKV_ALGO_TWO_PASS || o.static_scratch ||
                    (o.algo == RWKV_ALGO_AUTO && nTT <= kTwoPassMaxTiles);
    if (two_pass && chunk > tmax)
        return fail(RWKV_ERR_ARG, "the two-pass scan takes chunk_len up to %d for this input dtype and mode (got %d); "
                                  "longer chunks run in the single-launch scan", tmax, chunk);
    const int64_t tiles = B * ((C + kTileChannels - 1) / kTileChannels) * nTT;
    if (T > chunk && o.static_scratch && (size_t)tiles * kTileChannels * 16 > kStaticScratchBytes)
        return fail(RWKV_ERR_ARG, "%lld tiles need %zu bytes of scratch, more than the %zu this entry point holds "
                                  "(use the allocating entry point)", (long long)tiles,
                    (size_t)tiles * kTileChannels * 16, kStaticScratchBytes);
    if (T > chunk && o.workspace) {
        const size_t need = chunk_workspace_bytes(B, T, C, chunk);
        if (o.workspace_bytes < need)
            return fail(RWKV_ERR_ARG, "workspace of %zu bytes is smaller than the %zu needed", o.workspace_bytes,
                        need);
    }
    if (T > chunk) {
        // A captured launch replays with the arguments of its capture.  The single pass stamps
        // its look-back words with a per-launch epoch from the host, so a replay would accept
        // the previous replay's words; under capture AUTO takes the two-pass scan instead, which
        // needs no epoch, and the library-cached workspace (allocated on first use) is refused.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone) {
            if (o.algo == RWKV_ALGO_CHUNKED || chunk > tmax)
                return fail(RWKV_ERR_ARG, "the single-launch chunked scan (RWKV_ALGO_CHUNKED, or a chunk_len above "
                                          "%d) cannot be captured into a graph: its look-back is stamped per "
                                          "launch", tmax);
            if (!o.workspace && !o.static_scratch)
                return fail(RWKV_ERR_ARG, "a chunked scan under stream capture needs opts->workspace "
                                          "(the library-cached workspace is allocated on first use)");
            two_pass = true;
        }
    }
    ChunkWorkspace ws{};
    if (T > chunk && o.static_scratch) {  // the two-pass scan's aggregates only
        void *base = nullptr;
        rwkv_status s = static_scratch(&base);
        if (s != RWKV_OK) return s;
        ws.aggs = static_cast<float *>(base);
    } else if (T > chunk) {  // more than one tile per chain: the prefixes need scratch
        const size_t need = chunk_workspace_bytes(B, T, C, chunk);
        void *base = o.workspace;  // its size was checked above
        if (!base) {
            rwkv_status s = cached_workspace(need, stream, &base);
            if (s != RWKV_OK) return s;
        }
        chunk_workspace_carve(base, B, T, C, chunk, &ws);
        if (!two_pass) ws.epoch = next_epoch();
    }
    e = two_pass ? launch_chunked_2pass(a, chunk, ws, stream) : launch_chunked(a, chunk, ws, stream);
    if (e != hipSuccess) return hip_fail(e, two_pass ? "launch (two-pass chunked)" : "launch (chunked)");
    return ok();
}

}  // namespace

extern "C" {

rwkv_status rwkv4_wkv_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                              const void *k, const void *v, void *y, const float *state_in,
                              float *state_out, hipStream_t stream, const rwkv4_opts *opts) {
    Resolved o;
    rwkv_status s = resolve_opts(opts, &o);
    if (s != RWKV_OK) return s;
    ForwardArgs a{};
    a.B = B;
    a.T = T;
    a.C = C;
    a.w = w;
    a.u = u;
    a.k = k;
    a.v = v;
    a.r = o.r;
    a.y = y;
    a.state_in = state_in;
    a.state_out = state_out;
    a.mode = o.r ? MODE_GATED : MODE_PLAIN;
    return run_forward(a, o, stream);
}

rwkv_status rwkv4_wkv_step(int64_t B, int64_t C, const float *w, const float *u, const void *k,
                           const void *v, const void *r, void *y, float *state, rwkv_dtype in_dtype,
                           rwkv_dtype out_dtype, hipStream_t stream) {
    rwkv_status s;
    if ((s = check_dtype(in_dtype, "in_dtype")) != RWKV_OK) return s;
    if ((s = check_dtype(out_dtype, "out_dtype")) != RWKV_OK) return s;
    if (!state) return fail(RWKV_ERR_ARG, "state is required (read and updated in place)");
    if (!k || !v || !y) return fail(RWKV_ERR_ARG, "k, v and y are required");
    Resolved o;
    o.in_dtype = in_dtype;
    o.out_dtype = out_dtype;
    o.r = r;
    o.algo = RWKV_ALGO_SEQUENTIAL;
    ForwardArgs a{};
    a.B = B;
    a.T = 1;
    a.C = C;
    a.w = w;
    a.u = u;
    a.k = k;
    a.v = v;
    a.r = r;
    a.y = y;
    a.state_in = state;
    a.state_out = state;
    a.mode = r ? MODE_GATED : MODE_PLAIN;
    return run_forward(a, o, stream);
}

}  // extern "C"

namespace {

rwkv_status timemix_impl(int64_t B, int64_t T, int64_t C, const void *x, const void *x_prev, void *x_last,
                         const float *mix_k, const float *mix_v, const float *mix_r, const void *k, const void *v,
                         const float *w, const float *u, void *y, void *xk_out, void *xv_out,
                         const float *state_in, float *state_out, hipStream_t stream, const Resolved &o) {
    if (o.r) return fail(RWKV_ERR_ARG, "opts->r must be NULL for rwkv4_timemix_fused (r is the mixed x)");
    if (T > 0 && !x) return fail(RWKV_ERR_ARG, "x is required when T > 0");
    if (!mix_r) return fail(RWKV_ERR_ARG, "mix_r is required");
    if (xk_out && !mix_k) return fail(RWKV_ERR_ARG, "xk_out needs mix_k");
    if (xv_out && !mix_v) return fail(RWKV_ERR_ARG, "xv_out needs mix_v");
    const size_t ei = esize(o.in_dtype);
    const size_t act = (size_t)(B > 0 && T > 0 && C > 0 ? B * T * C : 0) * ei;
    const size_t row = (size_t)(B > 0 && C > 0 ? B * C : 0) * ei;
    if (overlap(xk_out, act, x, act) || overlap(xv_out, act, x, act) || overlap(xk_out, act, xv_out, act) ||
        overlap(x_last, row, x, act) || overlap(xk_out, act, k, act) || overlap(xv_out, act, v, act))
        return fail(RWKV_ERR_ARG, "an output of rwkv4_timemix_fused overlaps an input or another output");
    ForwardArgs a{};
    a.B = B;
    a.T = T;
    a.C = C;
    a.w = w;
    a.u = u;
    a.k = k;
    a.v = v;
    a.x = x;
    a.x_prev = x_prev;
    a.x_last = x_last;
    a.mix_r = mix_r;
    a.mix_k = mix_k ? mix_k : mix_r;  // unused unless xk_out is set
    a.mix_v = mix_v ? mix_v : mix_r;  // unused unless xv_out is set
    a.xk_out = xk_out;
    a.xv_out = xv_out;
    a.y = y;
    a.state_in = state_in;
    a.state_out = state_out;
    a.mode = MODE_TIMEMIX;
    return run_forward(a, o, stream);
}

}  // namespace

extern "C" {

rwkv_status rwkv4_timemix_fused(int64_t B, int64_t T, int64_t C, const void *x, const void *x_prev,
                                void *x_last, const float *mix_k, const float *mix_v,
                                const float *mix_r, const void *k, const void *v, const float *w,
                                const float *u, void *y, void *xk_out, void *xv_out,
                                const float *state_in, float *state_out, hipStream_t stream,
                                const rwkv4_opts *opts) {
    Resolved o;
    rwkv_status s = resolve_opts(opts, &o);
    if (s != RWKV_OK) return s;
    return timemix_impl(B, T, C, x, x_prev, x_last, mix_k, mix_v, mix_r, k, v, w, u, y, xk_out, xv_out, state_in,
                        state_out, stream, o);
}

rwkv_status rwkv4_timemix_fused_noalloc(int64_t B, int64_t T, int64_t C, const void *x, const void *x_prev,
                                        void *x_last, const float *mix_k, const float *mix_v,
                                        const float *mix_r, const void *k, const void *v, const float *w,
                                        const float *u, void *y, void *xk_out, void *xv_out,
                                        const float *state_in, float *state_out, hipStream_t stream,
                                        const rwkv4_opts *opts) {
    Resolved o;
    rwkv_status s = resolve_opts(opts, &o);
    if (s != RWKV_OK) return s;
    if (o.workspace)
        return fail(RWKV_ERR_ARG, "opts->workspace must be NULL: rwkv4_timemix_fused_noalloc uses its own static "
                                  "scratch");
    if (o.algo == RWKV_ALGO_CHUNKED)
        return fail(RWKV_ERR_ARG, "rwkv4_timemix_fused_noalloc runs the sequential kernel or the two-pass scan, "
                                  "not RWKV_ALGO_CHUNKED");
    o.static_scratch = true;
    return timemix_impl(B, T, C, x, x_prev, x_last, mix_k, mix_v, mix_r, k, v, w, u, y, xk_out, xv_out, state_in,
                        state_out, stream, o);
}

rwkv_status rwkv4_shift_mix(int64_t B, int64_t T, int64_t C, const void *x, const void *x_prev,
                            void *x_last, const float *ln_weight, const float *ln_bias, float ln_eps,
                            const float *mix_k, const float *mix_v, const float *mix_r, void *xk,
                            void *xv, void *xr, rwkv_dtype dtype, hipStream_t stream) {
    rwkv_status s;
    if ((s = check_dtype(dtype, "dtype")) != RWKV_OK) return s;
    if (B < 1 || C < 1 || T < 0)
        return fail(RWKV_ERR_ARG, "sizes must satisfy B >= 1, C >= 1, T >= 0 (got %lld, %lld, %lld)",
                    (long long)B, (long long)T, (long long)C);
    if (B > kMaxElems / C || (T > 0 && B * C > kMaxElems / T)) return fail(RWKV_ERR_ARG, "B*T*C too large");
    if (B * ((T + 2) / 3 + 1) > 0x7fffffffLL) return fail(RWKV_ERR_ARG, "B*T too large for one launch");
    if (T > 0 && !x) return fail(RWKV_ERR_ARG, "x is required when T > 0");
    if (!ln_weight && ln_bias) return fail(RWKV_ERR_ARG, "ln_bias is set but ln_weight is not");
    if (ln_weight && !(ln_eps >= 0.f && ln_eps <= 3.0e38f))
        return fail(RWKV_ERR_ARG, "ln_eps must be finite and >= 0");
    const float *mix[3] = {mix_k, mix_v, mix_r};
    void *out[3] = {xk, xv, xr};
    const char *names[3] = {"xk", "xv", "xr"};
    for (int i = 0; i < 3; ++i)  // with no tokens there is nothing to write (outputs may be NULL)
        if (T > 0 && (mix[i] == nullptr) != (out[i] == nullptr))
            return fail(RWKV_ERR_ARG, "%s and its mix must be given together", names[i]);
    const size_t e = esize(dtype);
    for (const void *p : {x, x_prev, (const void *)x_last, (const void *)xk, (const void *)xv, (const void *)xr})
        if (p && !aligned(p, e)) return fail(RWKV_ERR_ALIGN, "activation pointer %p not aligned to %zu bytes", p, e);
    for (const float *p : {ln_weight, ln_bias, mix_k, mix_v, mix_r})
        if (p && !aligned(p, 4)) return fail(RWKV_ERR_ALIGN, "fp32 pointer %p not 4-byte aligned", (const void *)p);
    const size_t act = (size_t)(B * T * C) * e, row = (size_t)(B * C) * e;
    for (int i = 0; i < 3; ++i) {
        if (overlap(out[i], act, x, act) || overlap(out[i], act, x_prev, row) || overlap(out[i], act, x_last, row))
            return fail(RWKV_ERR_ARG, "%s overlaps x, x_prev or x_last", names[i]);
        for (int j = i + 1; j < 3; ++j)
            if (overlap(out[i], act, out[j], act)) return fail(RWKV_ERR_ARG, "%s overlaps %s", names[i], names[j]);
    }
    if (overlap(x_last, row, x, act)) return fail(RWKV_ERR_ARG, "x_last overlaps x");
    if (x_last && x_prev && x_last != x_prev && overlap(x_last, row, x_prev, row))
        return fail(RWKV_ERR_ARG, "x_last overlaps x_prev without being equal to it");
    ShiftMixArgs a{};
    a.B = B;
    a.T = T;
    a.C = C;
    a.x = x;
    a.x_prev = x_prev;
    a.x_last = x_last;
    a.ln_weight = ln_weight;
    a.ln_bias = ln_bias;
    a.ln_eps = ln_eps;
    bool vec = (C % 8) == 0;
    for (int i = 0; i < 3; ++i) {
        a.mix[i] = T > 0 ? mix[i] : nullptr;
        a.out[i] = T > 0 ? out[i] : nullptr;
        if ((mix[i] && !aligned(mix[i], 16)) || (out[i] && !aligned(out[i], 16))) vec = false;
    }
    for (const void *p : {x, x_prev, (const void *)x_last, (const void *)ln_weight, (const void *)ln_bias})
        if (p && !aligned(p, 16)) vec = false;
    a.vec = vec ? 1 : 0;
    a.dt = dtype;
    if (T == 0 && !x_last) return ok();
    const hipError_t err = launch_shift_mix(a, stream);
    if (err != hipSuccess) return hip_fail(err, "launch (shift-mix)");
    return ok();
}

rwkv_status rwkv4_channelmix_gate(int64_t n, const void *r, const void *kv, const void *residual, void *y,
                                  rwkv_dtype in_dtype, rwkv_dtype out_dtype, hipStream_t stream) {
    rwkv_status s;
    if ((s = check_dtype(in_dtype, "in_dtype")) != RWKV_OK) return s;
    if ((s = check_dtype(out_dtype, "out_dtype")) != RWKV_OK) return s;
    if (n < 0 || n > kMaxElems) return fail(RWKV_ERR_ARG, "n must be in [0, 2^46] (got %lld)", (long long)n);
    if (n == 0) return ok();
    if (!r || !kv || !y) return fail(RWKV_ERR_ARG, "r, kv and y are required");
    const size_t ei = esize(in_dtype), eo = esize(out_dtype);
    for (const void *p : {r, kv, residual})
        if (p && !aligned(p, ei)) return fail(RWKV_ERR_ALIGN, "input pointer %p not aligned to %zu bytes", p, ei);
    if (!aligned(y, eo)) return fail(RWKV_ERR_ALIGN, "y not aligned to %zu bytes", eo);
    const size_t bi = (size_t)n * ei, bo = (size_t)n * eo;
    // y may be the residual itself (an in-place residual add: each element is read before it
    // is written by the same thread); no other overlap
    if (overlap(y, bo, r, bi) || overlap(y, bo, kv, bi) ||
        (residual && (y != residual || eo != ei) && overlap(y, bo, residual, bi)))
        return fail(RWKV_ERR_ARG, "y overlaps an input (only y == residual with equal dtypes is allowed)");
    GateLaunch g{};
    g.n = n;
    g.r = r;
    g.kv = kv;
    g.residual = residual;
    g.y = y;
    g.in_dt = in_dtype;
    g.out_dt = out_dtype;
    bool vec = (n % 8) == 0;
    for (const void *p : {r, kv, residual, (const void *)y})
        if (p && !aligned(p, 16)) vec = false;
    g.vec = vec ? 1 : 0;
    const hipError_t err = launch_gate(g, stream);
    if (err != hipSuccess) return hip_fail(err, "launch (channel-mix gate)");
    return ok();
}

const char *rwkv_status_string(rwkv_status s) {
    switch (s) {
        case RWKV_OK: return "ok";
        case RWKV_ERR_ARG: return "invalid argument";
        case RWKV_ERR_DTYPE: return "invalid dtype";
        case RWKV_ERR_ALIGN: return "misaligned pointer";
        case RWKV_ERR_HIP: return "HIP runtime error";
        case RWKV_ERR_NOMEM: return "out of device memory";
    }
    return "unknown status";
}

const char *rwkv_last_error(void) { return g_err; }

size_t rwkv4_workspace_bytes(int64_t B, int64_t T, int64_t C, int32_t chunk_len) {
    if (B < 1 || C < 1 || T < 1) return 0;
    // chunk_len 0: the size for the automatic choice whatever the dtype (64-token tiles, the
    // largest workspace; fp16 long sequences may then use 128-token tiles and need less)
    int chunk = chunk_len > 0 ? chunk_len : auto_chunk_len(B, T, C, 0);
    if (T <= chunk) return 0;
    return chunk_workspace_bytes(B, T, C, chunk);
}

rwkv_status rwkv4_lookback_status(void *workspace, hipStream_t stream, int32_t *gave_up) {
    if (!gave_up) return fail(RWKV_ERR_ARG, "gave_up is required");
    *gave_up = 0;
    if (workspace && !aligned(workspace, 256)) return fail(RWKV_ERR_ALIGN, "workspace must be 256-byte aligned");
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    void *base = workspace;
    if (!base) {
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        std::lock_guard<std::mutex> lk(g_ws_mu);
        const CachedWorkspace *w = find_cached(dev, stream);
        if (!w || !w->ptr) return ok();  // no chunked scan has run on this stream
        base = w->ptr;
    }
    uint32_t word = 0;
    e = hipMemcpy(&word, base, sizeof word, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    if (word != 0) {
        e = hipMemsetAsync(base, 0, sizeof word, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "clearing the error word");
        *gave_up = 1;
    }
    return ok();
}

int rwkv_abi_version(void) { return RWKV_ABI_VERSION; }

}  // extern "C"
