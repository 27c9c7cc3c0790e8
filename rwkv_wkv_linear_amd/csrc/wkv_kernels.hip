// wkv_kernels.hip -- gfx950 kernels for the RWKV-4 WKV time-mixing path.
//
// The recurrence (the WKV operator of the RWKV paper, arXiv 2305.13048, cited by
// the "RWKV-4 14B" page; the TR-2026-0009 port report, Methods and
// Reproducibility, carries it as a per-channel numerator/denominator/max state in
// fp32 with the max-trick).  Per channel the state is (a, b, p): numerator
// a * e^p and denominator b * e^p, where p tracks the largest log-weight so
// every exponential below has a non-positive argument:
//
//   output at token t:   q = max(p, u + k_t)
//                        wkv_t = (a e^{p-q} + v_t e^{u+k_t-q}) / (b e^{p-q} + e^{u+k_t-q})
//   absorb token t:      q = max(p + w, k_t)
//                        a <- a e^{p+w-q} + v_t e^{k_t-q};  b likewise with 1;  p <- q
//
// One of the two factors in each step is exactly 1, so each costs one
// exponential: e^{-|d|} with d the difference of the two candidates.
//
// The running max is kept as an anchor key and an age, p = key + n w: the largest
// term is always some token's key decayed n steps (or the prior state's pp).
// Every difference of candidates is then formed as (key - k_t) + (small terms),
// which is exact for nearby keys (Sterbenz), so the rounding of p does not grow
// with |k| or accumulate over steps as p <- p + w would.
//
// Spans compose: the state after a span of L tokens, started from s, is s aged by
// L merged with the span's own summary from the empty state, by the same max rule.
// This operator is associative, which the chunked scan uses to split T across
// lanes and workgroups.
//
// Kernels:
//   wkv_seq_kernel    one lane per (b, 4 channels), loops over T (large B*C, decode).
//   wkv_tile_kernel   one workgroup per (b, 64 channels, tile of TW tokens); each wave holds
//                     L tokens of the 64 channels, one lane per channel, in VGPRs from load
//                     to store.  A lane reduces its tokens to a summary, the waves fold the
//                     summaries in LDS, a decoupled look-back over earlier tiles supplies the
//                     tile's incoming state, and each lane replays its tokens to emit y.
//                     HBM traffic is one read of each input and one write of y.
//   wkv_passthrough   T = 0: copy the state (and x_prev to x_last).

#include "rwkvwkv.h"
#include "wkv_internal.h"

#ifndef RWKV_TU_IN
#error "compile with -DRWKV_TU_IN=0, 1 or 2 (the input dtype of this unit)"
#endif

#include <algorithm>
#include <mutex>
#include <vector>

namespace rwkvwkv {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEmptyP = -1.0e38f;  // p of the empty state (finite, so differences stay defined)
constexpr uint32_t kAgg = 1u, kIncl = 2u;
constexpr uint32_t kMaxSpins = 1u << 16;  // tens of milliseconds of polling (one memory round trip per spin) before a look-back gives up
constexpr int kMaxAnchorGap = 16;         // largest spacing of anchor tiles in a chain (a wave polls <= 4)

template <typename T> struct Raw;
template <> struct Raw<float> { using type = f4; };
template <> struct Raw<_Float16> { using type = h4; };
template <> struct Raw<__bf16> { using type = b4; };

__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

struct St {
    float a, b;  // numerator and denominator scaled by e^{-p}
    float k;     // anchor key of the largest term
    float n;     // its age in tokens: p = k + n * w
};

__device__ __forceinline__ St st_empty() { return St{0.f, 0.f, kEmptyP, 0.f}; }

// w = -inf (full forgetting) is carried as a large finite decay, so that 0 * w stays 0;
// e^{-1e30} and e^{-inf} are both exactly 0 in fp32.
__device__ __forceinline__ float finite_decay(float w) { return fmaxf(w, -1.0e30f); }

__device__ __forceinline__ St st_load(float aa, float bb, float pp) { return St{aa, bb, pp, 0.f}; }
__device__ __forceinline__ float st_logmax(const St &s, float w) { return fmaf(s.n, w, s.k); }

// State s, then L tokens whose own summary (from the empty state) is t.
__device__ __forceinline__ St combine(const St &s, const St &t, float L, float w) {
    const float d = (s.k - t.k) + (s.n + L - t.n) * w;  // p_s + L w - p_t
    const float e = ex(-fabsf(d));
    const bool left = d >= 0.f;
    const float e1 = left ? 1.f : e, e2 = left ? e : 1.f;
    return St{s.a * e1 + t.a * e2, s.b * e1 + t.b * e2, left ? s.k : t.k, left ? s.n + L : t.n};
}

// Absorb token (k, v).
__device__ __forceinline__ void absorb(St &s, float w, float k, float v) {
    const float n1 = s.n + 1.f;
    const float d = fmaf(n1, w, s.k - k);  // p + w - k
    const float e = ex(-fabsf(d));
    const bool left = d >= 0.f;
    const float e1 = left ? 1.f : e, e2 = left ? e : 1.f;
    s.a = s.a * e1 + v * e2;
    s.b = s.b * e1 + e2;
    s.k = left ? s.k : k;
    s.n = left ? n1 : 0.f;
}

// Numerator and denominator of the output at token (k, v) with bonus u.
__device__ __forceinline__ void emit(const St &s, float w, float u, float k, float v, float &num,
                                     float &den) {
    const float d = (s.k - k) + fmaf(s.n, w, -u);  // p - (u + k)
    const float e = ex(-fabsf(d));
    const bool left = d >= 0.f;
    const float e1 = left ? 1.f : e, e2 = left ? e : 1.f;
    num = s.a * e1 + v * e2;
    den = s.b * e1 + e2;
}

// Four consecutive channels at element offset `off`; nch of them valid.  With vec
// set, nch is 0 or 4 and the access is one aligned vector load.
// Activations and states are read once per launch: the loads are streaming (non-temporal)
// hints, so they do not displace reused lines (parameters, published tile states) from L2.
template <typename T>
__device__ __forceinline__ typename Raw<T>::type load4(const T *p, int64_t off, int nch, bool vec) {
    using R = typename Raw<T>::type;
    R r = {0, 0, 0, 0};
    if (vec) {
        if (nch == 4) r = __builtin_nontemporal_load(reinterpret_cast<const R *>(p + off));
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nch) r[q] = __builtin_nontemporal_load(p + off + q);
    }
    return r;
}

// Every output of these kernels is written once and never read back by the launch that writes
// it: streaming (non-temporal) stores keep the written lines from lingering dirty in L2, where
// the end-of-kernel write-back would otherwise flush them after the last workgroup.
template <typename V>
__device__ __forceinline__ void st_stream(V *p, V v) {
    __builtin_nontemporal_store(v, p);
}

template <typename T>
__device__ __forceinline__ void store4(T *p, int64_t off, int nch, bool vec, const float (&x)[4]) {
    using R = typename Raw<T>::type;
    if (vec) {
        if (nch == 4) {
            R r;
#pragma unroll
            for (int q = 0; q < 4; ++q) r[q] = (T)x[q];  // fp16: round to nearest even
            st_stream(reinterpret_cast<R *>(p + off), r);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nch) st_stream(p + off + q, (T)x[q]);
    }
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane l's
// bytes land at lds + 16 l.  `lds` must be the same for the whole wave.  The rows are read
// once: cache policy 2 is the non-temporal (streaming) hint.
__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 2);
}

// L values of one channel, one per token, as loaded.
template <typename T, int L> struct Rows {
    T p[L];
    __device__ __forceinline__ float get(int i) const { return (float)p[i]; }
};

// Four per-channel parameters c0 .. c0+3 (zeros past C); one 16-byte load when aligned.
__device__ __forceinline__ void load_param4(const float *p, int64_t c0, int nch, bool vec, float (&x)[4]) {
    if (vec && nch == 4) {
        const f4 v = *reinterpret_cast<const f4 *>(p + c0);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = v[q];
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = (q < nch) ? p[c0 + q] : 0.f;
}

// ------------------------------------------------------------------------------------------
// Sequential kernel: lane = (b, channels c0..c0+3), loop over T.

template <typename TIn, typename TOut, int MODE>
__global__ void __launch_bounds__(256) wkv_seq_kernel(ForwardArgs a) {
    const int64_t ngroups = (a.C + 3) / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.B * ngroups) return;
    const int64_t b = gid / ngroups;
    const int64_t c0 = (gid - b * ngroups) * 4;
    const int nch = (int)std::min<int64_t>(4, a.C - c0);
    const bool vec = a.vec != 0;
    const int64_t BC = a.B * a.C, sc = b * a.C + c0;

    const TIn *K = static_cast<const TIn *>(a.k);
    const TIn *V = static_cast<const TIn *>(a.v);
    TOut *Y = static_cast<TOut *>(a.y);

    float w[4], u[4];
    const bool vp = a.vecp != 0;
    load_param4(a.w, c0, nch, vp, w);
    load_param4(a.u, c0, nch, vp, u);
    St s[4];
    const bool vs = a.vecs != 0 && nch == 4;  // the lane's state is three aligned float4
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = finite_decay(w[q]);
    if (a.state_in && vs) {
        const f4 A = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.state_in + sc));
        const f4 Bq = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.state_in + BC + sc));
        const f4 P = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(a.state_in + 2 * BC + sc));
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] = st_load(A[q], Bq[q], P[q]);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] = st_empty();
            if (a.state_in && q < nch)
                s[q] = st_load(a.state_in[sc + q], a.state_in[BC + sc + q], a.state_in[2 * BC + sc + q]);
        }
    }
    float mk[4], mv[4], mr[4], xs[4];
    if constexpr (MODE == MODE_TIMEMIX) {
        load_param4(a.mix_k, c0, nch, vp, mk);
        load_param4(a.mix_v, c0, nch, vp, mv);
        load_param4(a.mix_r, c0, nch, vp, mr);
        const TIn *XP = static_cast<const TIn *>(a.x_prev);
        auto xp = XP ? load4(XP, sc, nch, vec) : typename Raw<TIn>::type{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) xs[q] = (float)xp[q];
    }

    const int64_t row0 = b * a.T * a.C + c0;
#pragma unroll 2
    for (int64_t t = 0; t < a.T; ++t) {
        const int64_t off = row0 + t * a.C;
        const auto kr = load4(K, off, nch, vec);
        const auto vr = load4(V, off, nch, vec);
        typename Raw<TIn>::type gr = {0, 0, 0, 0};
        if constexpr (MODE == MODE_GATED) gr = load4(static_cast<const TIn *>(a.r), off, nch, vec);
        if constexpr (MODE == MODE_TIMEMIX) gr = load4(static_cast<const TIn *>(a.x), off, nch, vec);
        float yv[4], xko[4], xvo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float kk = (float)kr[q], vv = (float)vr[q];
            float num, den;
            emit(s[q], w[q], u[q], kk, vv, num, den);
            float g = 1.f;
            if constexpr (MODE == MODE_GATED) g = 1.f + ex(-(float)gr[q]);
            if constexpr (MODE == MODE_TIMEMIX) {
                const float xx = (float)gr[q];
                const float xr = mr[q] * xx + (1.f - mr[q]) * xs[q];
                xko[q] = mk[q] * xx + (1.f - mk[q]) * xs[q];
                xvo[q] = mv[q] * xx + (1.f - mv[q]) * xs[q];
                xs[q] = xx;
                g = 1.f + ex(-xr);
            }
            yv[q] = num * rcp(den * g);
            absorb(s[q], w[q], kk, vv);
        }
        store4(Y, off, nch, vec, yv);
        if constexpr (MODE == MODE_TIMEMIX) {
            if (a.xk_out) store4(static_cast<TIn *>(a.xk_out), off, nch, vec, xko);
            if (a.xv_out) store4(static_cast<TIn *>(a.xv_out), off, nch, vec, xvo);
        }
    }
    if (a.state_out && vs) {
        f4 A, Bq, P;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            A[q] = s[q].a;
            Bq[q] = s[q].b;
            P[q] = st_logmax(s[q], w[q]);
        }
        st_stream(reinterpret_cast<f4 *>(a.state_out + sc), A);
        st_stream(reinterpret_cast<f4 *>(a.state_out + BC + sc), Bq);
        st_stream(reinterpret_cast<f4 *>(a.state_out + 2 * BC + sc), P);
    } else if (a.state_out) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nch) {
                st_stream(a.state_out + sc + q, s[q].a);
                st_stream(a.state_out + BC + sc + q, s[q].b);
                st_stream(a.state_out + 2 * BC + sc + q, st_logmax(s[q], w[q]));
            }
    }
    if constexpr (MODE == MODE_TIMEMIX) {
        if (a.x_last) store4(static_cast<TIn *>(a.x_last), sc, nch, vec, xs);
    }
}

// ------------------------------------------------------------------------------------------
// Chunked scan.

// Cross-workgroup exchange.  Each published state field is one 64-bit word: the fp32
// value in the low half, the tag (epoch << 2 | kind) in the high half, written and read
// as relaxed agent-scope 64-bit atomics.  A reader accepts a tile's state when all four of
// its words carry the expected tag, so no fence (and no L2 write-back or invalidate) is
// needed: each word is self-validating and the fields need no mutual order.
// With local set the words are stored at workgroup scope: they stay in this XCD's L2, where the
// device-scope loads of a reader on the same XCD find them without a trip to memory (a reader
// on another XCD cannot see them until they are stored again at device scope).  Otherwise they
// are written through to memory at once.
__device__ __forceinline__ void publish(const ChunkWorkspace &ws, int64_t tile, uint32_t kind,
                                        const St &s, int ch, bool local) {
    uint64_t *dst = ws.words + tile * (4 * kTileChannels);
    const uint64_t tag = (uint64_t)((ws.epoch << 2) | kind) << 32;
    const float f[4] = {s.a, s.b, s.k, s.n};
    if (local) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            __hip_atomic_store(dst + m * kTileChannels + ch, tag | __float_as_uint(f[m]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            __hip_atomic_store(dst + m * kTileChannels + ch, tag | __float_as_uint(f[m]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Fold of the published states of tiles [lo, hi) of a chain, left to right; tile lo is an
// anchor (inclusive state) when lo_incl is set, every other tile an aggregate.  Every lane
// loads its channel's fields of every tile and checks every tag; while some are missing the
// wave reads all of them again, back to back (a state found in the same XCD's L2 costs one
// short round trip, so a separate probe word followed by a second full read would only add one).
// The workspace's error word is read with the first attempt and every 64th after it: once a
// wait on the workspace has given up, every later wait gives up at once, in this launch and in
// later ones, until the caller reads and clears the word (rwkv4_lookback_status).  A wait gives
// up after kMaxSpins attempts too; it then stores the launch's epoch in the error word and
// returns NaNs, so the failure shows in the outputs as well.
template <int MAXT>
__device__ St fold_published(const ChunkWorkspace &ws, int64_t chain, int64_t lo, int64_t hi, bool lo_incl,
                             float wc, float TW, int ch) {
    const int cnt = (int)(hi - lo);
    const uint32_t want_agg = (ws.epoch << 2) | kAgg, want_incl = (ws.epoch << 2) | kIncl;
    uint64_t w[MAXT][4] = {};  // slots past cnt are never loaded; their checks are masked
    const uint64_t *tiles = ws.words + (chain + lo) * (4 * kTileChannels);  // wave-uniform
    // The words of every tile are requested before any is checked: with each tile's check next
    // to its loads, the compiler waited for that tile's words before requesting the next
    // tile's, one memory round trip per predecessor on every poll.  Only the cnt tiles in use
    // are read (the polls share the memory channels with the publishes they wait for).
    auto read_all = [&]() -> bool {
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
            if (m < cnt) {
                const uint64_t *src = tiles + m * (4 * kTileChannels) + ch;
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    w[m][f] = __hip_atomic_load(src + f * kTileChannels, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        uint32_t ok = 1u;
#pragma unroll
        for (int m = 0; m < MAXT; ++m) {
            const uint32_t want = (m == 0 && lo_incl) ? want_incl : want_agg;
            uint32_t tm = 1u;
#pragma unroll
            for (int f = 0; f < 4; ++f) tm &= (uint32_t)((uint32_t)(w[m][f] >> 32) == want);
            ok &= tm | (uint32_t)(m >= cnt);
        }
        return __all(ok != 0u);
    };
    // one read site (a second inlined copy of read_all would hold a second set of words)
    bool failed = false;
    for (uint32_t spins = 0;; ++spins) {
        const bool check = (spins & 63u) == 0u;
        uint32_t e = 0;
        if (check) e = __hip_atomic_load(ws.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // with the reads
        const bool done = read_all();
        if ((check && __builtin_amdgcn_readfirstlane(e) != 0u) || (!done && spins >= kMaxSpins)) {
            failed = true;
            break;
        }
        if (done) break;
    }
    if (failed) {
        __hip_atomic_store(ws.err, ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return St{__builtin_nanf(""), __builtin_nanf(""), 0.f, 0.f};
    }
    St acc = st_empty();
#pragma unroll
    for (int m = 0; m < MAXT; ++m) {
        if (m < cnt) {
            const St x = St{__uint_as_float((uint32_t)w[m][0]), __uint_as_float((uint32_t)w[m][1]),
                            __uint_as_float((uint32_t)w[m][2]), __uint_as_float((uint32_t)w[m][3])};
            acc = (m == 0) ? x : combine(acc, x, TW, wc);
        }
    }
    return acc;
}

// Linear-space fast path of the tile kernel.  Within one wave's L tokens a lane scales every
// weight by e^{-kmax}, kmax the largest key of its tokens; the weights e^{k_i - kmax} are then
// at most 1, computed once, and the numerator/denominator run as plain fp32 recurrences
// (n <- e^w n + X v).  The guard keeps every surviving term a normal fp32 number:
//   key spread kmax - kmin <= 40 nats (the summary and the emit): every weight lies in
//   [e^-40, 1], or in [e^-40, e^40] when the staged summary scales by its first group's
//   largest key;
//   bonus -20 <= u <= 30 (the emit): each current-token weight e^{u + k_t - kmax} is at least
//   e^{-60}, so anything flushed to zero is < 1e-12 of it, and at most e^70 (fp32 overflows
//   past e^88);
//   incoming state scale p - kmax <= 60 (the emit), so it cannot overflow.
// A lane outside the guard runs the exact per-token max-trick instead (same results within
// rounding; the tests drive both paths, and waves whose lanes take different paths).
// Workgroups are handed to the eight XCDs round-robin by index, so blockIdx % 8 picks a
// workgroup's XCD.  When nCT is a multiple of 8, the plain order (r = b * nCT + ct) gives each
// XCD every eighth chain, all in the same 128-byte column of every 1 KB of each row, and the
// column at bytes 384-511 loads about a sixth slower on MI355X (measured: the slowness moves
// with the column, not the XCD), so one XCD ends well after the rest.  Index r then goes to
// chain (r % 8) * (B * nCT / 8) + r / 8 instead: each XCD runs a contiguous range of chains
// that spans all columns.  With rot set (calls of more workgroups than the GPU holds at once)
// the ranges also rotate over the XCDs from one time tile to the next, (r + tt) % 8 in place
// of r % 8; otherwise every time tile of a chain runs on one XCD.  Measured: rotation takes
// the B1 T65536 C2048 call from 252 to 237 us and costs a one-round call (the 14B layer) 1.5
// us.  When nCT is not a multiple of 8, consecutive batch rows already shift the column an XCD
// sees, and the plain order stays (measured faster there).
__device__ __forceinline__ void tile_chain(int64_t rem, int64_t tt, int rot, int64_t BCT, int nCT, int64_t &b,
                                           int64_t &ct) {
    constexpr int kXcds = 8;
    const int64_t r = (nCT % kXcds == 0) ? ((rem + (rot ? tt : 0)) % kXcds) * (BCT / kXcds) + rem / kXcds : rem;
    b = r / nCT;
    ct = r - b * nCT;
}

// How a tile gets its incoming state: from its predecessors in the same launch (single
// pass, decoupled look-back) or from tile aggregates a previous launch wrote (two passes).
constexpr int PREFIX_LOOKBACK = 0, PREFIX_AGGS = 1;

// LDS one workgroup may hold on gfx950 (the CU's 160 KB).
constexpr size_t kTileLdsMax = 160 * 1024;

// Longest chunk the single-launch scan stages in LDS as one tile: NT tensors of rows plus the
// wave summaries, waves of 32 tokens (2-byte inputs, up to 16 waves ungated and 8 otherwise)
// or 16 (fp32, up to 16 waves).
template <typename TIn, int MODE>
constexpr int staged_tile_max() {
    constexpr int NT = MODE == MODE_PLAIN ? 2 : 3;
    constexpr int L = sizeof(TIn) == 2 ? 32 : 16;
    constexpr int maxS = (L == 32 && MODE != MODE_PLAIN) ? 8 : 16;
    int S = maxS;
    while (S > 4 && (size_t)NT * S * L * kTileChannels * sizeof(TIn) + (size_t)4 * S * kTileChannels * 4 > kTileLdsMax)
        S /= 2;
    return S * L;
}

constexpr float kGuardSpread = 40.f;
constexpr float kGuardBonus = -20.f;
constexpr float kGuardBonusMax = 30.f;
constexpr float kGuardState = 60.f;

// Phase A of a tile: wave wv stages its L rows (tokens t0 .. t0+L-1 of the tile) of each
// of the NT tensors in src into LDS rows[NT][TW][64].  With 16-byte vectors (vec16) each
// global_load_lds_dwordx4 moves RPI whole 128-B (fp16) or 256-B (fp32) rows, no VGPR holds
// a load in flight, and the instructions go out RPI rows of every tensor at a time (the
// staged summary waits for them group by group); otherwise each lane loads its own channel in rolled batches of 4 rows (a
// rare path, kept from setting the kernel's register footprint).  Rows past T and chunks past
// C read a valid clamped address whose data is never used.
template <typename TIn, int NT, int L>
__device__ __forceinline__ void stage_rows(const TIn *const *src, TIn *rows, int TW, int wv, int lane, int64_t b,
                                           int64_t T, int64_t C, int64_t ct, int64_t tile_t0, int64_t t0,
                                           int64_t cs, bool vec16) {
    constexpr int CW = kTileChannels;
    if (vec16) {
        constexpr int CH16 = 16 / (int)sizeof(TIn);  // channels per 16-byte chunk
        constexpr int CHUNKS = CW / CH16;           // chunks per row: 8 (fp16) or 16 (fp32)
        constexpr int RPI = 64 / CHUNKS;            // rows per instruction: 8 or 4
        const int q = lane % CHUNKS, rsub = lane / CHUNKS;
        int64_t cq = ct * CW + q * CH16;
        if (cq >= C) cq = 0;
        // row-group major (rows j*RPI .. of every tensor, then the next rows): loads complete
        // in issue order, so the summary can take each group of rows as it lands
#pragma unroll
        for (int j = 0; j < L / RPI; ++j) {
#pragma unroll
            for (int tsr = 0; tsr < NT; ++tsr) {
                const int r = wv * L + j * RPI;
                const int64_t t = std::min<int64_t>(tile_t0 + r + rsub, T - 1);
                dma16(src[tsr] + (b * T + t) * C + cq, rows + ((size_t)tsr * TW + r) * CW);
            }
        }
    } else {
        const int64_t tl = std::min<int64_t>(t0, T - 1);
        const int last = (int)std::min<int64_t>(L - 1, T - 1 - tl);
#pragma unroll
        for (int tsr = 0; tsr < NT; ++tsr) {
            const TIn *col = src[tsr] + (b * T + tl) * C + cs;
#pragma unroll 1
            for (int i0 = 0; i0 < L; i0 += 4) {
                TIn tmp[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) tmp[i] = col[(int64_t)std::min(i0 + i, last) * C];
#pragma unroll
                for (int i = 0; i < 4; ++i) rows[((size_t)tsr * TW + wv * L + i0 + i) * CW + lane] = tmp[i];
            }
        }
    }
}

// Phase B of a tile: the summary of one wave's nval tokens from the empty state (kr, vr point
// at the lane's first staged key and value).  Padded tokens (i >= nval) get weight X = 0 and
// decay 1, so they leave every recurrence unchanged.  Sets kmax (the largest key) and fast
// (whether the key-spread part of the linear-space guard holds; else the exact per-token max-trick ran).
template <typename TIn, int L>
__device__ __forceinline__ St wave_summary(const TIn *kr, const TIn *vr, int nval, float wc, float uc, float ew,
                                           float &kmax, bool &fast, float (&Xs)[L]) {
    constexpr int CW = kTileChannels;
    kmax = -INFINITY;
    float kmin = INFINITY;
    St sum = st_empty();
    float xk[L], vb[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        xk[i] = (float)kr[i * CW];
        vb[i] = (float)vr[i * CW];
    }
    if (nval == L) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            kmax = fmaxf(kmax, xk[i]);
            kmin = fminf(kmin, xk[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            kmax = fmaxf(kmax, i < nval ? xk[i] : -INFINITY);
            kmin = fminf(kmin, i < nval ? xk[i] : INFINITY);
        }
    }
    fast = nval > 0 && (kmax - kmin) <= kGuardSpread;
    if (fast) {
        float nn = 0.f, dd = 0.f;
        if (nval == L) {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const float X = ex(xk[i] - kmax);
                Xs[i] = X;  // kept for the emit phase
                nn = fmaf(ew, nn, X * vb[i]);
                dd = fmaf(ew, dd, X);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const float X = (i < nval) ? ex(xk[i] - kmax) : 0.f;
                const float e = (i < nval) ? ew : 1.f;
                nn = fmaf(e, nn, X * vb[i]);
                dd = fmaf(e, dd, X);
            }
        }
        sum = St{nn, dd, kmax, 0.f};
    } else {
#pragma unroll
        for (int i = 0; i < L; ++i)
            if (i < nval) absorb(sum, wc, xk[i], vb[i]);
    }
    return sum;
}

// Wait until at most N vector-memory instructions of this wave are outstanding (gfx9
// s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Phase B for a full wave whose rows arrive by 16-byte DMA in row-group order (stage_rows):
// the summary takes 8 tokens at a time as soon as they have landed, while the later groups are
// still in flight.  Weights are scaled by the largest key of the first group, mref, instead of
// the wave's largest key (unknown until the last group lands): with the key spread of the wave
// at most kGuardSpread every weight e^{k - mref} stays a normal fp32 number, and the guard is
// decided after the last group exactly as in wave_summary.  Loads complete in issue order, so
// when at most (instructions issued after group g) are outstanding, group g is in LDS: only
// the k and v rows may be in flight when it is called.
template <typename TIn, int L>
__device__ __forceinline__ St wave_summary_staged(const TIn *kr, const TIn *vr, float ew, float uc, float &mref,
                                                  bool &fast, float (&Xs)[L]) {
    constexpr int CW = kTileChannels, G = 8, NG = L / G;
    constexpr int RPI = 64 / (CW / (16 / (int)sizeof(TIn)));  // rows per DMA instruction
    constexpr int IPG = 2 * (G / RPI);                        // DMA instructions per group (k, v)
    static_assert(L % G == 0 && G % RPI == 0, "groups are whole DMA instructions");
    float nn = 0.f, dd = 0.f, kmax = -INFINITY, kmin = INFINITY, m = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (NG - 1 - g == 3) wait_vmcnt<3 * IPG>();
        else if (NG - 1 - g == 2) wait_vmcnt<2 * IPG>();
        else if (NG - 1 - g == 1) wait_vmcnt<IPG>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_wave_barrier();
        float xk[G], vb[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            xk[i] = (float)kr[(g * G + i) * CW];
            vb[i] = (float)vr[(g * G + i) * CW];
        }
        float gmax = xk[0], gmin = xk[0];
#pragma unroll
        for (int i = 1; i < G; ++i) {
            gmax = fmaxf(gmax, xk[i]);
            gmin = fminf(gmin, xk[i]);
        }
        if (g == 0) m = gmax;
        kmax = fmaxf(kmax, gmax);
        kmin = fminf(kmin, gmin);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float X = ex(xk[i] - m);
            Xs[g * G + i] = X;  // kept for the emit phase
            nn = fmaf(ew, nn, X * vb[i]);
            dd = fmaf(ew, dd, X);
        }
    }
    static_assert(NG <= 4, "at most four groups per wave");
    fast = (kmax - kmin) <= kGuardSpread;
    mref = m;
    return St{nn, dd, m, 0.f};
}

// Linear-space emit of one wave's L tokens when all of them are valid: y_i from the running
// numerator/denominator (nn, dd, scaled by e^{-kmax}), then the recurrence step.  With
// P = X v the four updates are single FMAs: num = nn + e^u P, den = dd + e^u X,
// nn <- e^w nn + P, dd <- e^w dd + X.  The optional writes are template switches so the
// unrolled loop has no branches: STAGE puts y in LDS, rows [0, L/2) at ystage_lo and rows
// [L/2, L) at ystage_hi, and writes every finished batch of rows with 16-byte stores (yrow
// 16-byte aligned, all 64 channels in range).  The staging rows are the wave's dead k rows and
// its v rows; a v row is read into registers at the start of its batch, before any y row that
// overlaps it is written (an output twice the input's size covers input rows 2(i - L/2) and
// 2(i - L/2) + 1 with output row i >= L/2, all at or before i).  MIX
// writes the time-mix xk/xv rows.  Xs holds the weights e^{k_i - kmax} from the summary
// phase; vr, gr point at the lane's first staged row.  The gate factor is 1 + e^{-r_i}
// (r_i = mr x_i + (1 - mr) x_{i-1} for the time mix, in base 2 as ga x_i + gb x_{i-1}).
template <typename TIn, typename TOut, int MODE, int L, bool STAGE, bool MIX>
__device__ __forceinline__ void emit_full(const float (&Xs)[L], const TIn *vr, const TIn *gr,
                                          float eu, float ew, float ga, float gb, float mk, float mv, float &xs,
                                          float &nn, float &dd, TOut *yrow, TIn *xkrow, TIn *xvrow, TOut *ystage_lo,
                                          TOut *ystage_hi,
                                          unsigned Cu, int lane) {
    constexpr int CW = kTileChannels;
    constexpr int LB = 8;  // rows read from LDS per batch, to bound the registers they occupy
    // products with a +0 addend keep fp16 operands in a mixed-precision FMA (no separate
    // conversion); they round exactly like the plain product
    float gbx = gb * xs;  // the gate's previous-token term
#pragma unroll
    for (int h = 0; h < L; h += LB) {
        TIn vh[LB], gh[LB];
        constexpr bool kNeedX = MODE != MODE_PLAIN;  // x (or r) rows read here
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            vh[j] = vr[(h + j) * CW];
            gh[j] = kNeedX ? gr[(h + j) * CW] : TIn(0);
        }
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            const int i = h + j;
            const float X = Xs[i];  // e^{k_i - kmax} from the summary phase
            const float P = fmaf(X, (float)vh[j], 0.f);
            const float num = fmaf(eu, P, nn);
            const float den = fmaf(eu, X, dd);
            float dg = den;  // den * (1 + e^{-r})
            if constexpr (MODE == MODE_GATED) dg = fmaf(den, __builtin_amdgcn_exp2f(-kLog2e * (float)gh[j]), den);
            if constexpr (MODE == MODE_TIMEMIX) {
                dg = fmaf(den, __builtin_amdgcn_exp2f(fmaf(ga, (float)gh[j], gbx)), den);
                if constexpr (MIX) {
                    const float xx = (float)gh[j];
                    const unsigned off = i * Cu + (unsigned)lane;
                    if (xkrow) st_stream(xkrow + off, (TIn)fmaf(mk, xx - xs, xs));
                    if (xvrow) st_stream(xvrow + off, (TIn)fmaf(mv, xx - xs, xs));
                    xs = xx;
                }
                gbx = fmaf(gb, (float)gh[j], 0.f);
            }
            const TOut yv = (TOut)(num * rcp(dg));
            if constexpr (STAGE)
                (i < L / 2 ? ystage_lo + i * CW : ystage_hi + (i - L / 2) * CW)[lane] = yv;
            else
                st_stream(yrow + i * Cu + (unsigned)lane, yv);
            nn = fmaf(ew, nn, P);
            dd = fmaf(ew, dd, X);
        }
        if constexpr (STAGE) {
            // rows h .. h+LB-1 of y are complete in LDS: write them as 16-byte chunks now, so the
            // stores overlap the rest of the emit instead of leaving all at its end
            __builtin_amdgcn_wave_barrier();
            constexpr int CH16 = 16 / (int)sizeof(TOut);  // outputs per 16-byte chunk
            constexpr int CHUNKS = CW / CH16;
            constexpr int RPI = 64 / CHUNKS;             // rows per store instruction
            static_assert(LB % RPI == 0, "a batch is a whole number of store instructions");
            // the halves are apart only for an output wider than the input (RPI 4); the rows of
            // one store instruction then lie in one half
            static_assert(sizeof(TOut) <= sizeof(TIn) || (L / 2) % RPI == 0, "one half per store");
            const int q = lane % CHUNKS, rs = lane / CHUNKS;
#pragma unroll
            for (int j = 0; j < LB / RPI; ++j) {
                const int r = h + j * RPI + rs;
                const TOut *ys = h + j * RPI < L / 2 ? ystage_lo + r * CW : ystage_hi + (r - L / 2) * CW;
                const f4 chunk = *reinterpret_cast<const f4 *>(ys + q * CH16);
                st_stream(reinterpret_cast<f4 *>(yrow + r * Cu + q * CH16), chunk);
            }
        }
    }
    if constexpr (MODE == MODE_TIMEMIX && !MIX) xs = (float)gr[(L - 1) * CW];
}

// Phase B of a tile: the summary of the wave's tokens from the empty state, with only this
// wave's k and v rows in flight.  A full wave whose rows come by 16-byte DMA takes them group by
// group as they land (wave-uniform choice); lanes past C then drop their summary (their rows
// are a copy of channel 0), and lanes outside the key-spread guard redo it exactly.  Otherwise
// the wave waits for its rows and runs wave_summary.
template <typename TIn, int L>
__device__ __forceinline__ St summarize_wave(const TIn *kr, const TIn *vr, int wlen, int nval, bool cok, bool vec16,
                                             float wc, float uc, float ew, float &kmax, bool &fast, float (&Xs)[L]) {
    constexpr int CW = kTileChannels;
    St sum;
    if (vec16 && wlen == L) {
        sum = wave_summary_staged<TIn, L>(kr, vr, ew, uc, kmax, fast, Xs);
        if (!cok) {
            sum = st_empty();
            fast = false;
        } else if (!fast) {
            // outside the linear-space guard: the exact per-token recurrence (all rows landed)
            sum = st_empty();
#pragma unroll 1
            for (int i = 0; i < L; ++i) absorb(sum, wc, (float)kr[i * CW], (float)vr[i * CW]);
        }
    } else {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed in LDS
        __builtin_amdgcn_wave_barrier();
        sum = wave_summary<TIn, L>(kr, vr, nval, wc, uc, ew, kmax, fast, Xs);
    }
    return sum;
}

// Phase E of a tile: emit y (and the time mix's xk, xv) for the wave's tokens starting from the
// state st, and return the state after them.  kr, vr, gr point at the lane's first staged key,
// value and gate row, krow0 and vrow0 at the wave's first k and v rows (y is staged there); Xs holds the weights
// of the linear-space summary (fast), kmax their reference key; xs is the time mix's previous
// token, updated to the wave's last.  base is the element offset of the lane's first token.
template <typename TIn, typename TOut, int MODE, int L>
__device__ __forceinline__ St emit_wave(const ForwardArgs &a, const St &st, const float (&Xs)[L], bool fast,
                                        float kmax, const TIn *kr, const TIn *vr, const TIn *gr, TIn *krow0,
                                        TIn *vrow0,
                                        float wc, float uc, float ew, float eu, float ga, float gb, float mk,
                                        float mv, float &xs, int64_t b, int64_t ct, int64_t t0, int wlen, int nval,
                                        int64_t base, int lane) {
    constexpr int CW = kTileChannels;
    const int64_t C = a.C;
    TOut *Y = static_cast<TOut *>(a.y);
    TIn *XKO = static_cast<TIn *>(a.xk_out);
    TIn *XVO = static_cast<TIn *>(a.xv_out);
    const float pst = st_logmax(st, wc);
    // the lane's tokens take the linear-space path; a wave whose lanes all do may stage y
    const bool lane_fast = fast && pst - kmax <= kGuardState && uc >= kGuardBonus && uc <= kGuardBonusMax;
    const bool wave_fast = __all(lane_fast);  // voted before the lanes diverge
    St fin;
    if (lane_fast) {
        const float s0 = ex(pst - kmax);
        float nn = st.a * s0, dd = st.b * s0;
        // rows as wave-uniform pointers plus a 32-bit lane offset
        const int64_t row0 = (b * a.T + t0) * C + ct * CW;
        const unsigned Cu = (unsigned)C;
        // a full wave (all L tokens, all 64 channels in range, every lane on this path) stages y
        // in LDS and writes 16 bytes per lane: each lane's store carries other lanes' channels,
        // so no lane may be on the exact path.  y rows up to the input's size go in the wave's v
        // rows, dead once read; twice that size in its k rows (first half) and v rows
        constexpr bool kStageFits = sizeof(TOut) <= 2 * sizeof(TIn);
        const bool stage_y = kStageFits && wlen == L && ct * CW + CW <= C && a.vec16y && a.vec16 && wave_fast;
        TOut *ystage_lo = reinterpret_cast<TOut *>(sizeof(TOut) > sizeof(TIn) ? krow0 : vrow0);
        TOut *ystage_hi = sizeof(TOut) > sizeof(TIn) ? reinterpret_cast<TOut *>(vrow0) : ystage_lo + (L / 2) * CW;
        if (nval == L) {
            const bool mix = (MODE == MODE_TIMEMIX) && (XKO || XVO);
            TOut *yrow = Y + row0;
            TIn *xkrow = XKO ? XKO + row0 : nullptr, *xvrow = XVO ? XVO + row0 : nullptr;
#define RWKV_EMIT(STAGE, MIX)                                                                          \
    emit_full<TIn, TOut, MODE, L, STAGE, MIX>(Xs, vr, gr, eu, ew, ga, gb, mk, mv, xs, nn, dd, yrow, \
                                                   xkrow, xvrow, ystage_lo, ystage_hi, Cu, lane)
            if constexpr (MODE == MODE_TIMEMIX) {
                if (stage_y) {
                    if (mix) RWKV_EMIT(true, true); else RWKV_EMIT(true, false);
                } else {
                    if (mix) RWKV_EMIT(false, true); else RWKV_EMIT(false, false);
                }
            } else {
                if (stage_y) RWKV_EMIT(true, false); else RWKV_EMIT(false, false);
            }
#undef RWKV_EMIT
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const float kk = (float)kr[i * CW], vv = (float)vr[i * CW];
                const float X = (i < nval) ? ex(kk - kmax) : 0.f;
                const float XU = X * eu;
                const float num = fmaf(XU, vv, nn);
                const float den = dd + XU;
                float g = 1.f;
                float xx = 0.f;
                if constexpr (MODE == MODE_GATED) g = 1.f + __builtin_amdgcn_exp2f(-kLog2e * (float)gr[i * CW]);
                if constexpr (MODE == MODE_TIMEMIX) {
                    xx = (float)gr[i * CW];
                    g = 1.f + __builtin_amdgcn_exp2f(fmaf(ga, xx, gb * xs));
                }
                const float yv = num * rcp(den * g);
                if (i < nval) {
                    st_stream(Y + base + i * C, (TOut)yv);
                    if constexpr (MODE == MODE_TIMEMIX) {
                        if (XKO) st_stream(XKO + base + i * C, (TIn)fmaf(mk, xx - xs, xs));
                        if (XVO) st_stream(XVO + base + i * C, (TIn)fmaf(mv, xx - xs, xs));
                    }
                }
                if constexpr (MODE == MODE_TIMEMIX) xs = (i < nval) ? xx : xs;
                const float e = (i < nval) ? ew : 1.f;
                nn = fmaf(e, nn, X * vv);
                dd = fmaf(e, dd, X);
            }
        }
        fin = St{nn, dd, kmax, 0.f};
    } else {
        // exact per-token max-trick
        St s2 = st;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if (i < nval) {
                const float kk = (float)kr[i * CW];
                const float vv = (float)vr[i * CW];
                float num, den;
                emit(s2, wc, uc, kk, vv, num, den);
                float g = 1.f;
                if constexpr (MODE == MODE_GATED) g = 1.f + ex(-(float)gr[i * CW]);
                if constexpr (MODE == MODE_TIMEMIX) {
                    const float xx = (float)gr[i * CW];
                    g = 1.f + __builtin_amdgcn_exp2f(fmaf(ga, xx, gb * xs));
                    if (XKO) st_stream(XKO + base + i * C, (TIn)fmaf(mk, xx - xs, xs));
                    if (XVO) st_stream(XVO + base + i * C, (TIn)fmaf(mv, xx - xs, xs));
                    xs = xx;
                }
                st_stream(Y + base + i * C, (TOut)(num * rcp(den * g)));
                absorb(s2, wc, kk, vv);
            }
        }
        fin = s2;
    }
    return fin;
}

// Workgroup = (b, channel tile ct of 64 channels, time tile tt of TW = S * L tokens),
// blockIdx = tt * (B * nCT) + r with (b, ct) = tile_chain(r), so every tile a workgroup waits
// for has a lower index and was dispatched earlier.  PREFIX selects where the tile's incoming state
// comes from: the single-pass look-back (phase D) or the aggregates of a first pass.  Wave w of S = tokens tt*TW + w*L .. +L-1;
// lane = channel ct*64 + lane.
//
// The tile's rows of k, v (and r or x) are staged in LDS as [tensor][TW][64] by 16-byte
// global-to-LDS loads (global_load_lds_dwordx4): each wave fetches the L rows it computes
// on, 8 rows of 128 B per instruction, so no VGPR holds a load in flight and a wave waits
// only for its own rows.  When the pointers are not
// 16-byte aligned or C is not a multiple of a 16-byte chunk, each lane loads its own
// channel instead (same LDS layout).  Rows past T and chunks past C read a valid address
// whose data is never used.  A full wave keeps its weights X_i from phase B to phase E
// (saving an exponential per token); amdgpu_waves_per_eu(5) holds the kernel to 96 VGPRs,
// so with 28 KB of LDS five workgroups share a CU and every workgroup of a layer-sized
// call is resident at once.
template <typename TIn, typename TOut, int MODE, int L, int PREFIX>
__device__ __forceinline__ void tile_body(const ForwardArgs &a, const ChunkWorkspace &ws, int S, int nCT, int nTT,
                                          int TW, int M, int rot, int lp, int G) {
    constexpr int CW = kTileChannels;
    constexpr int NT = (MODE == MODE_PLAIN) ? 2 : 3;  // staged tensors: k, v, [r | x]
    extern __shared__ __attribute__((aligned(16))) char smem[];
    TIn *rows = reinterpret_cast<TIn *>(smem);                                  // [NT][TW][CW]
    float *sF = reinterpret_cast<float *>(smem + (size_t)NT * TW * CW * sizeof(TIn));  // [4][S][CW]
    float *sI = sF;  // [4][S][CW] parts of the incoming state, once every wave has read sF

    // wv is the same in every lane of a wave: readfirstlane lets the compiler keep
    // wave-uniform row and tile addresses in SGPRs
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t BCT = a.B * nCT;
    const int64_t tt = blockIdx.x / G;  // G workgroups per time tile: the BCT chains, then padding
    const int64_t rem = blockIdx.x - tt * G;
    if (rem >= BCT) return;
    // Until its emit a wave runs at raised issue priority: its summary and publish are on the
    // critical path of the chain's later tiles, while the emit of a tile whose prefix has arrived
    // is not, and at the end of a launch the two compete for the same SIMDs.
    __builtin_amdgcn_s_setprio(2);
    int64_t b, ct;
    tile_chain(rem, tt, rot, BCT, nCT, b, ct);
    const int64_t c = ct * CW + lane;
    const bool cok = c < a.C;
    const int64_t tile_t0 = tt * TW;
    const int64_t tile_len = std::min<int64_t>(TW, a.T - tile_t0);
    const int64_t t0 = tile_t0 + (int64_t)wv * L;
    const int wlen = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - t0));  // tokens of this wave
    const int nval = cok ? wlen : 0;
    const int64_t C = a.C, BC = a.B * a.C;
    const int64_t base = (b * a.T + t0) * C + c;
    const int64_t cs = cok ? c : 0;  // loads stay unpredicated: a lane past C reads channel 0

    const TIn *K = static_cast<const TIn *>(a.k);
    const TIn *V = static_cast<const TIn *>(a.v);
    const TIn *GR = static_cast<const TIn *>(MODE == MODE_GATED ? a.r : a.x);

    const int64_t chain = (b * nCT + ct) * nTT;

    // Two passes: the aggregates of tiles 0 .. tt-1 are complete before this launch.  Wave wv
    // loads its share (issued before the row loads, so it lands first) and folds it, wave 0
    // starting from state_in; the shares are combined in order through LDS while the rows are
    // still in flight.  The result is state_in + AGG(0) + ... + AGG(tt-1), folded in a fixed
    // order.
    St prefix = st_empty();
    St part = st_empty();
    int q = 0;
    if constexpr (PREFIX == PREFIX_AGGS) {
        if (tt > 0) {
            q = (int)((tt + S - 1) / S);
            const int lo = wv * q, hi = std::min<int>(lo + q, (int)tt);
            const f4 *src = reinterpret_cast<const f4 *>(ws.aggs) + (chain + lo) * CW + lane;
            bool have = false;
            if (wv == 0 && a.state_in && cok) {
                part = st_load(a.state_in[b * C + c], a.state_in[BC + b * C + c], a.state_in[2 * BC + b * C + c]);
                have = true;
            }
            const float w_pre = finite_decay(a.w[cs]);
            for (int j0 = lo; j0 < hi; j0 += 4) {
                f4 x[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (j0 + m < hi) x[m] = src[(j0 - lo + m) * CW];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (j0 + m < hi) {
                        const St g = St{x[m][0], x[m][1], x[m][2], x[m][3]};
                        part = have ? combine(part, g, (float)TW, w_pre) : g;
                        have = true;
                    }
            }
        }
    }

    // Per-channel parameters, the time-mix token before the tile and the prior state are loaded
    // before the rows: vector loads complete in issue order, so they are in registers before the
    // first group of rows, and the staged summary's counted waits see only the row loads after
    // them.  The empty asm keeps the compiler from moving memory accesses across it.
    const float w_raw = a.w[cs], u_raw = a.u[cs];
    const float wc = cok ? finite_decay(w_raw) : 0.f;
    const float uc = cok ? u_raw : 0.f;
    float xs = 0.f, mr = 0.f, mk = 0.f, mv = 0.f;
    if constexpr (MODE == MODE_TIMEMIX) {
        // the token before the wave's first: x[t0 - 1], or x_prev (zeros if absent) at t0 = 0; a
        // wave past T reads a valid address it does not use
        const bool from_x = t0 > 0 && t0 <= a.T, from_prev = t0 == 0 && a.x_prev != nullptr;
        const TIn *xsrc = from_prev ? static_cast<const TIn *>(a.x_prev) + b * C + cs
                                    : GR + (from_x ? (b * a.T + t0 - 1) * C + cs : 0);
        const float xv = (float)*xsrc;
        const float mr_raw = a.mix_r[cs], mk_raw = a.mix_k[cs], mv_raw = a.mix_v[cs];
        xs = (from_x || from_prev) ? xv : 0.f;
        mr = cok ? mr_raw : 0.f;
        mk = cok ? mk_raw : 0.f;
        mv = cok ? mv_raw : 0.f;
    }
    if (tt == 0 && a.state_in && cok)
        prefix = st_load(a.state_in[b * C + c], a.state_in[BC + b * C + c], a.state_in[2 * BC + b * C + c]);
    asm volatile("" ::: "memory");

    // Phase A: stage this wave's k and v rows.  The r (or x) rows feed only the gate in the emit,
    // so they are requested after the summary (phase B), behind the k and v rows of every
    // workgroup, and land while the look-back runs: the summaries, and so the published
    // aggregates, do not wait for a third of the bytes.
    const TIn *src[3] = {K, V, GR};
    stage_rows<TIn, 2, L>(src, rows, TW, wv, lane, b, a.T, C, ct, tile_t0, t0, cs, a.vec16 != 0);
    const float ew = ex(wc), eu = ex(uc);
    // gate argument in base 2: -log2(e) * (mr x + (1 - mr) xs)
    const float ga = -kLog2e * mr, gb = -kLog2e * (1.f - mr);
    if (PREFIX == PREFIX_AGGS && tt > 0) {
        sF[(0 * S + wv) * CW + lane] = part.a;
        sF[(1 * S + wv) * CW + lane] = part.b;
        sF[(2 * S + wv) * CW + lane] = part.k;
        sF[(3 * S + wv) * CW + lane] = part.n;
        lds_barrier();
        for (int j = 0; j < S; ++j) {
            const int lj = j * q;
            if (lj < (int)tt) {
                const St pj = St{sF[(0 * S + j) * CW + lane], sF[(1 * S + j) * CW + lane],
                                 sF[(2 * S + j) * CW + lane], sF[(3 * S + j) * CW + lane]};
                const float span = (float)((std::min(lj + q, (int)tt) - lj) * TW);
                prefix = (j == 0) ? pj : combine(prefix, pj, span, wc);
            }
        }
        lds_barrier();  // the wave summaries reuse sF next
    }
    const TIn *kr = rows + ((size_t)0 * TW + wv * L) * CW + lane;
    const TIn *vr = rows + ((size_t)1 * TW + wv * L) * CW + lane;
    const TIn *gr = rows + ((size_t)2 * TW + wv * L) * CW + lane;

    // Phase B: summary of the wave's tokens from the empty state; then the wave requests its
    // gate rows.
    float kmax;   // the weights' reference key: the largest key (or the first group's, staged)
    bool fast;
    float Xs[L];  // the weights e^{k_i - kmax} of a full wave on the fast path
    const St sum = summarize_wave<TIn, L>(kr, vr, wlen, nval, cok, a.vec16 != 0, wc, uc, ew, kmax, fast, Xs);
    if constexpr (NT == 3)  // waited for before the emit
        stage_rows<TIn, 1, L>(src + 2, rows + (size_t)2 * TW * CW, TW, wv, lane, b, a.T, C, ct, tile_t0, t0, cs,
                              a.vec16 != 0);
    sF[(0 * S + wv) * CW + lane] = sum.a;
    sF[(1 * S + wv) * CW + lane] = sum.b;
    sF[(2 * S + wv) * CW + lane] = sum.k;
    sF[(3 * S + wv) * CW + lane] = sum.n;
    lds_barrier();  // not waiting for the gate rows in flight

    // Phase C: each wave folds the summaries of the waves before it (fixed order); the last
    // wave forms the tile aggregate and publishes it.
    St excl = st_empty();
    for (int j = 0; j < wv; ++j) {
        const St sj = St{sF[(0 * S + j) * CW + lane], sF[(1 * S + j) * CW + lane],
                         sF[(2 * S + j) * CW + lane], sF[(3 * S + j) * CW + lane]};
        const int lj = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - (tile_t0 + (int64_t)j * L)));
        excl = combine(excl, sj, (float)lj, wc);
    }
    const bool anchor = (tt % M) == 0, last = tt == nTT - 1;
    St agg = st_empty();
    if constexpr (PREFIX == PREFIX_LOOKBACK) {
        if (wv == S - 1) {
            agg = combine(excl, sum, (float)wlen, wc);
            if (nTT > 1 && !anchor && !last) publish(ws, chain + tt, kAgg, agg, lane, lp != 0);
        }
    }

    // Phase D: the tile's incoming state.  Anchor tiles (every M-th, tile 0 included) publish
    // their inclusive state, the others only their aggregate; with a the last anchor before tt
    // the prefix is INCL(a) + AGG(a+1) + ... + AGG(tt-1), folded in that fixed order whatever
    // the timing, so results are bitwise reproducible.  The waves share the polling: wave w
    // folds a contiguous part, then every wave folds the parts in order.
    if (PREFIX == PREFIX_LOOKBACK && tt > 0) {
        const int a0 = (int)(((tt - 1) / M) * M);
        const int cnt = (int)tt - a0;
        q = (cnt + S - 1) / S;
        const int lo = a0 + wv * q, hi = std::min(lo + q, (int)tt);
        if (lo < hi) part = fold_published<kMaxAnchorGap / 4>(ws, chain, lo, hi, lo == a0, wc, (float)TW, lane);
        lds_barrier();  // sI reuses sF: every wave has folded its summaries (phase C)
        sI[(0 * S + wv) * CW + lane] = part.a;
        sI[(1 * S + wv) * CW + lane] = part.b;
        sI[(2 * S + wv) * CW + lane] = part.k;
        sI[(3 * S + wv) * CW + lane] = part.n;
        lds_barrier();
        for (int j = 0; j < S; ++j) {
            const int lj = a0 + j * q;
            if (lj < (int)tt) {
                const St pj = St{sI[(0 * S + j) * CW + lane], sI[(1 * S + j) * CW + lane],
                                 sI[(2 * S + j) * CW + lane], sI[(3 * S + j) * CW + lane]};
                const float span = (float)((std::min(lj + q, (int)tt) - lj) * TW);
                prefix = (j == 0) ? pj : combine(prefix, pj, span, wc);
            }
        }
    }
    // an anchor's inclusive state does not wait for the gate rows: the chain's later tiles fold it
    if (PREFIX == PREFIX_LOOKBACK && wv == S - 1 && nTT > 1 && anchor && !last) {
        agg = combine(prefix, agg, (float)tile_len, wc);  // from here on the published (inclusive) state
        publish(ws, chain + tt, kIncl, agg, lane, lp != 0);
    }
    if constexpr (NT == 3) {
        // this wave's gate rows have landed; the emit reads no other wave's (each wave loaded the
        // token before its first itself), so a wave starts as soon as its own rows are in
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
    }
    const St st = combine(prefix, excl, (float)std::min<int64_t>((int64_t)wv * L, tile_len), wc);

    // Phase E: emit y for the wave's tokens, starting from st.
    __builtin_amdgcn_s_setprio(0);
    const St fin = emit_wave<TIn, TOut, MODE, L>(a, st, Xs, fast, kmax, kr, vr, gr,
                                                 rows + ((size_t)0 * TW + wv * L) * CW,
                                                 rows + ((size_t)1 * TW + wv * L) * CW, wc, uc, ew, eu, ga, gb,
                                                 mk, mv, xs, b, ct, t0, wlen, nval, base, lane);

    // A state published into this XCD's L2 is now written through for readers on other XCDs
    // (the outputs above are out of the way).
    if (PREFIX == PREFIX_LOOKBACK && lp && wv == S - 1 && nTT > 1 && !last)
        publish(ws, chain + tt, anchor ? kIncl : kAgg, agg, lane, false);

    // Phase F: the lane holding token T-1 writes the final state (and x_last).
    if (nval > 0 && t0 + nval == a.T) {
        if (a.state_out) {
            st_stream(a.state_out + b * C + c, fin.a);
            st_stream(a.state_out + BC + b * C + c, fin.b);
            st_stream(a.state_out + 2 * BC + b * C + c, st_logmax(fin, wc));
        }
        if constexpr (MODE == MODE_TIMEMIX) {
            if (a.x_last) st_stream(static_cast<TIn *>(a.x_last) + b * C + c, (TIn)xs);
        }
    }
}

// Long tiles: chunk_len CL above the longest tile staged in LDS at once (staged_tile_max), in
// sub-tiles of SUBW = S * L tokens (4 waves of L tokens: 128 tokens for 2-byte inputs, 64 for
// fp32).  A workgroup owns CL tokens of a chain as
// NSUB = CL / SUBW consecutive sub-tiles that pass one after another through the same LDS rows.
// Pass 1 folds every sub-tile's wave summaries into the chunk's aggregate, which the tile
// publishes for the later tiles of its chain (the last tile of a chain, which nothing waits
// for, skips it); after the look-back, whose words now cover CL tokens each, pass 2 stages
// each sub-tile again and emits it from the running state, as tile_body does for one tile.
// The k and v rows are read twice, the second time shortly after the first (so mostly from
// L2 or the Infinity Cache).  States are published straight to memory (write-through).
template <typename TIn, typename TOut, int MODE, int L>
__device__ __forceinline__ void long_tile_body(const ForwardArgs &a, const ChunkWorkspace &ws, int S, int nCT,
                                               int nTT, int CL, int M, int rot, int G) {
    constexpr int CW = kTileChannels;
    constexpr int NT = (MODE == MODE_PLAIN) ? 2 : 3;  // staged tensors: k, v, [r | x]
    const int SUBW = S * L;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    TIn *rows = reinterpret_cast<TIn *>(smem);                                          // [NT][SUBW][CW]
    float *sF = reinterpret_cast<float *>(smem + (size_t)NT * SUBW * CW * sizeof(TIn));  // [4][S][CW]

    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t BCT = a.B * nCT;
    const int64_t tt = blockIdx.x / G;
    const int64_t rem = blockIdx.x - tt * G;
    if (rem >= BCT) return;
    __builtin_amdgcn_s_setprio(2);  // pass 1 and the look-back feed the chain's later tiles
    int64_t b, ct;
    tile_chain(rem, tt, rot, BCT, nCT, b, ct);
    const int64_t c = ct * CW + lane;
    const bool cok = c < a.C;
    const int64_t C = a.C, BC = a.B * a.C;
    const int64_t cs = cok ? c : 0;  // loads stay unpredicated: a lane past C reads channel 0
    const int64_t chunk_t0 = tt * CL;
    const int64_t chunk_len = std::min<int64_t>(CL, a.T - chunk_t0);
    const int nsub = (int)((chunk_len + SUBW - 1) / SUBW);
    const int64_t chain = (b * nCT + ct) * nTT;
    const bool vec16 = a.vec16 != 0;

    const TIn *K = static_cast<const TIn *>(a.k);
    const TIn *V = static_cast<const TIn *>(a.v);
    const TIn *GR = static_cast<const TIn *>(MODE == MODE_GATED ? a.r : a.x);
    const TIn *src[3] = {K, V, GR};

    const float w_raw = a.w[cs], u_raw = a.u[cs];
    const float wc = cok ? finite_decay(w_raw) : 0.f;
    const float uc = cok ? u_raw : 0.f;
    float mr = 0.f, mk = 0.f, mv = 0.f;
    if constexpr (MODE == MODE_TIMEMIX) {
        const float mr_raw = a.mix_r[cs], mk_raw = a.mix_k[cs], mv_raw = a.mix_v[cs];
        mr = cok ? mr_raw : 0.f;
        mk = cok ? mk_raw : 0.f;
        mv = cok ? mv_raw : 0.f;
    }
    St prefix = st_empty();
    if (tt == 0 && a.state_in && cok)
        prefix = st_load(a.state_in[b * C + c], a.state_in[BC + b * C + c], a.state_in[2 * BC + b * C + c]);
    asm volatile("" ::: "memory");
    const float ew = ex(wc), eu = ex(uc);
    const float ga = -kLog2e * mr, gb = -kLog2e * (1.f - mr);
    const TIn *kr = rows + ((size_t)0 * SUBW + wv * L) * CW + lane;
    const TIn *vr = rows + ((size_t)1 * SUBW + wv * L) * CW + lane;
    const TIn *gr = rows + ((size_t)2 * SUBW + wv * L) * CW + lane;

    const bool anchor = (tt % M) == 0, last = tt == nTT - 1;
    const bool publishes = nTT > 1 && !last;

    // Pass 1: the chunk's aggregate, from the empty state (only a tile that publishes needs it).
    // Each wave stages and summarises its own rows; wave S-1 folds the waves' summaries of every
    // sub-tile in token order.
    St agg = st_empty();
    if (publishes) {
#pragma unroll 1
        for (int j = 0; j < nsub; ++j) {
            const int64_t sub_t0 = chunk_t0 + (int64_t)j * SUBW;
            const int64_t t0 = sub_t0 + (int64_t)wv * L;
            const int wlen = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - t0));
            stage_rows<TIn, 2, L>(src, rows, SUBW, wv, lane, b, a.T, C, ct, sub_t0, t0, cs, vec16);
            float kmax;
            bool fast;
            float Xs[L];
            const St sum = summarize_wave<TIn, L>(kr, vr, wlen, cok ? wlen : 0, cok, vec16, wc, uc, ew, kmax, fast, Xs);
            sF[(0 * S + wv) * CW + lane] = sum.a;
            sF[(1 * S + wv) * CW + lane] = sum.b;
            sF[(2 * S + wv) * CW + lane] = sum.k;
            sF[(3 * S + wv) * CW + lane] = sum.n;
            lds_barrier();
            if (wv == S - 1) {
                for (int q = 0; q < S; ++q) {
                    const St sq = St{sF[(0 * S + q) * CW + lane], sF[(1 * S + q) * CW + lane],
                                     sF[(2 * S + q) * CW + lane], sF[(3 * S + q) * CW + lane]};
                    const int lq = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - (sub_t0 + (int64_t)q * L)));
                    agg = combine(agg, sq, (float)lq, wc);
                }
            }
            lds_barrier();  // sF and the rows are rewritten by the next sub-tile
        }
        if (wv == S - 1 && !anchor) publish(ws, chain + tt, kAgg, agg, lane, false);
    }

    // The chunk's incoming state, as tile_body's phase D: INCL(a0) + AGG(a0+1) + ... + AGG(tt-1)
    // in that fixed order, the polling shared by the waves.
    if (tt > 0) {
        const int a0 = (int)(((tt - 1) / M) * M);
        const int cnt = (int)tt - a0;
        const int q = (cnt + S - 1) / S;
        const int lo = a0 + wv * q, hi = std::min(lo + q, (int)tt);
        St part = st_empty();
        if (lo < hi) part = fold_published<kMaxAnchorGap / 4>(ws, chain, lo, hi, lo == a0, wc, (float)CL, lane);
        sF[(0 * S + wv) * CW + lane] = part.a;
        sF[(1 * S + wv) * CW + lane] = part.b;
        sF[(2 * S + wv) * CW + lane] = part.k;
        sF[(3 * S + wv) * CW + lane] = part.n;
        lds_barrier();
        for (int j = 0; j < S; ++j) {
            const int lj = a0 + j * q;
            if (lj < (int)tt) {
                const St pj = St{sF[(0 * S + j) * CW + lane], sF[(1 * S + j) * CW + lane],
                                 sF[(2 * S + j) * CW + lane], sF[(3 * S + j) * CW + lane]};
                const float span = (float)((int64_t)(std::min(lj + q, (int)tt) - lj) * CL);
                prefix = (j == 0) ? pj : combine(prefix, pj, span, wc);
            }
        }
        lds_barrier();  // sF is rewritten in pass 2
    }
    if (publishes && anchor && wv == S - 1) publish(ws, chain + tt, kIncl, combine(prefix, agg, (float)chunk_len, wc), lane, false);

    // Pass 2: each sub-tile staged again and emitted from the running state.
    __builtin_amdgcn_s_setprio(0);
    St running = prefix;
    float xs = 0.f;
#pragma unroll 1
    for (int j = 0; j < nsub; ++j) {
        const int64_t sub_t0 = chunk_t0 + (int64_t)j * SUBW;
        const int64_t sub_len = std::min<int64_t>(SUBW, a.T - sub_t0);
        const int64_t t0 = sub_t0 + (int64_t)wv * L;
        const int wlen = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - t0));
        const int nval = cok ? wlen : 0;
        const int64_t base = (b * a.T + t0) * C + c;
        if constexpr (MODE == MODE_TIMEMIX) {
            // wave 0: x[sub_t0 - 1] or x_prev (zeros if absent); later waves read it from LDS
            if (wv == 0) {
                const bool from_x = sub_t0 > 0, from_prev = sub_t0 == 0 && a.x_prev != nullptr;
                const TIn *xsrc = from_prev ? static_cast<const TIn *>(a.x_prev) + b * C + cs
                                            : GR + (from_x ? (b * a.T + sub_t0 - 1) * C + cs : 0);
                const float xv = (float)*xsrc;
                xs = (from_x || from_prev) ? xv : 0.f;
            }
            asm volatile("" ::: "memory");
        }
        stage_rows<TIn, 2, L>(src, rows, SUBW, wv, lane, b, a.T, C, ct, sub_t0, t0, cs, vec16);
        float kmax;
        bool fast;
        float Xs[L];
        const St sum = summarize_wave<TIn, L>(kr, vr, wlen, nval, cok, vec16, wc, uc, ew, kmax, fast, Xs);
        if constexpr (NT == 3)  // waited for before the emit
            stage_rows<TIn, 1, L>(src + 2, rows + (size_t)2 * SUBW * CW, SUBW, wv, lane, b, a.T, C, ct, sub_t0, t0,
                                  cs, vec16);
        sF[(0 * S + wv) * CW + lane] = sum.a;
        sF[(1 * S + wv) * CW + lane] = sum.b;
        sF[(2 * S + wv) * CW + lane] = sum.k;
        sF[(3 * S + wv) * CW + lane] = sum.n;
        lds_barrier();  // not waiting for the gate rows in flight
        // every wave folds the waves before it (its exclusive prefix) and all of them (the
        // sub-tile's aggregate, which carries the running state to the next sub-tile)
        St excl = st_empty(), sub_agg = st_empty();
        for (int q = 0; q < S; ++q) {
            const St sq = St{sF[(0 * S + q) * CW + lane], sF[(1 * S + q) * CW + lane],
                             sF[(2 * S + q) * CW + lane], sF[(3 * S + q) * CW + lane]};
            const int lq = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - (sub_t0 + (int64_t)q * L)));
            if (q < wv) excl = combine(excl, sq, (float)lq, wc);
            sub_agg = combine(sub_agg, sq, (float)lq, wc);
        }
        if constexpr (NT == 3) {
            __builtin_amdgcn_s_waitcnt(0);  // this wave's gate rows have landed,
            __syncthreads();                // and every other wave's (the time mix reads the previous wave's last x)
        }
        const St st = combine(running, excl, (float)std::min<int64_t>((int64_t)wv * L, sub_len), wc);
        if constexpr (MODE == MODE_TIMEMIX) {
            if (wv > 0) xs = (float)gr[-CW];  // the previous wave's last row
        }
        // the emit's per-token output offsets (token x C + lane) are the same in every sub-tile;
        // an opaque copy of the lane index keeps the compiler from hoisting all of them out of
        // the loop, where they would hold a register each for the whole loop
        int lane_it = lane;
        asm volatile("" : "+v"(lane_it));
        const St fin = emit_wave<TIn, TOut, MODE, L>(a, st, Xs, fast, kmax, kr, vr, gr,
                                                     rows + ((size_t)0 * SUBW + wv * L) * CW,
                                                     rows + ((size_t)1 * SUBW + wv * L) * CW, wc, uc, ew, eu, ga,
                                                     gb, mk, mv, xs, b, ct, t0, wlen, nval, base, lane_it);
        running = combine(running, sub_agg, (float)sub_len, wc);
        // the lane holding token T-1 writes the final state (and x_last)
        if (nval > 0 && t0 + nval == a.T) {
            if (a.state_out) {
                st_stream(a.state_out + b * C + c, fin.a);
                st_stream(a.state_out + BC + b * C + c, fin.b);
                st_stream(a.state_out + 2 * BC + b * C + c, st_logmax(fin, wc));
            }
            if constexpr (MODE == MODE_TIMEMIX) {
                if (a.x_last) st_stream(static_cast<TIn *>(a.x_last) + b * C + c, (TIn)xs);
            }
        }
        lds_barrier();  // every wave is done with sF and with the rows it reads of other waves
    }
}

// Long tiles of 32-token waves (2-byte inputs, sub-tiles of 128 tokens) and of 16-token waves
// (fp32 inputs, sub-tiles of 64 tokens).  The sub-tile loop holds more registers than one tile:
// 32-token waves get up to 168 VGPRs (three waves per SIMD; two for the time mix, 256), 16-token
// waves up to 128.
template <typename TIn, typename TOut, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == MODE_TIMEMIX ? 2 : 3)))
    wkv_long32_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int CL, int M, int rot, int G) {
    long_tile_body<TIn, TOut, MODE, 32>(a, ws, S, nCT, nTT, CL, M, rot, G);
}

template <typename TIn, typename TOut, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
    wkv_long16_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int CL, int M, int rot, int G) {
    long_tile_body<TIn, TOut, MODE, 16>(a, ws, S, nCT, nTT, CL, M, rot, G);
}

// 16 tokens per wave (chunk_len = 16 * waves): 96 VGPRs so that five 4-wave workgroups
// share a CU.
template <typename TIn, typename TOut, int MODE, int PREFIX>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(5)))
    wkv_tile_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW, int M, int rot, int lp, int G) {
    tile_body<TIn, TOut, MODE, 16, PREFIX>(a, ws, S, nCT, nTT, TW, M, rot, lp, G);
}

// 8 tokens per wave: 32-token tiles of 4 waves, 16-token tiles of 2.
template <typename TIn, typename TOut, int MODE, int PREFIX>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5)))
    wkv_tile8_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW, int M, int rot, int lp, int G) {
    tile_body<TIn, TOut, MODE, 8, PREFIX>(a, ws, S, nCT, nTT, TW, M, rot, lp, G);
}

// 32 tokens per wave in 4 waves (128-token tiles): half as many tiles per chain, so a
// quarter of the look-back reads; three 52 KB workgroups share a CU, and with that
// occupancy each wave may hold its 32 weights in registers.  Up to 8 waves (256-token tiles).
template <typename TIn, typename TOut, int MODE, int PREFIX>
__global__ void __launch_bounds__(512)
    wkv_tile32_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW, int M, int rot, int lp, int G) {
    tile_body<TIn, TOut, MODE, 32, PREFIX>(a, ws, S, nCT, nTT, TW, M, rot, lp, G);
}

// 16 waves of 32 tokens (512-token tiles, ungated only: the k and v rows fill 128 KB of LDS).
template <typename TIn, typename TOut, int MODE, int PREFIX>
__global__ void __launch_bounds__(1024)
    wkv_tile32w_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW, int M, int rot, int lp, int G) {
    static_assert(MODE == MODE_PLAIN, "16 waves of staged gate rows do not fit in LDS");
    tile_body<TIn, TOut, MODE, 32, PREFIX>(a, ws, S, nCT, nTT, TW, M, rot, lp, G);
}

// ------------------------------------------------------------------------------------------

// First pass of the two-pass scan: the aggregate (summary from the empty state) of every
// time tile but the last of each chain, written as one float4 (a, b, key, age) per (tile,
// channel) to ws.aggs.  Same tiling and phases A-B as wkv_tile_kernel, on k and v only.
template <typename TIn, int L>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(5)))
    wkv_tile_agg_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW) {
    constexpr int CW = kTileChannels;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    TIn *rows = reinterpret_cast<TIn *>(smem);                                  // [2][TW][CW]
    float *sF = reinterpret_cast<float *>(smem + (size_t)2 * TW * CW * sizeof(TIn));  // [4][S][CW]
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t BCT = a.B * nCT;
    const int64_t tt = blockIdx.x / BCT;  // < nTT - 1: every tile here is full
    const int64_t rem = blockIdx.x - tt * BCT;
    int64_t b, ct;
    tile_chain(rem, tt, 0, BCT, nCT, b, ct);
    const int64_t c = ct * CW + lane;
    const bool cok = c < a.C;
    const int64_t tile_t0 = tt * TW, t0 = tile_t0 + (int64_t)wv * L;
    const int64_t cs = cok ? c : 0;
    {
        const TIn *src[2] = {static_cast<const TIn *>(a.k), static_cast<const TIn *>(a.v)};
        stage_rows<TIn, 2, L>(src, rows, TW, wv, lane, b, a.T, a.C, ct, tile_t0, t0, cs, a.vec16 != 0);
    }
    const float w_raw = a.w[cs], u_raw = a.u[cs];
    const float wc = cok ? finite_decay(w_raw) : 0.f;
    const float uc = cok ? u_raw : 0.f;
    const float ew = ex(wc);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    float kmax;
    bool fast;
    float Xs[L];
    const St sum = wave_summary<TIn, L>(rows + (size_t)wv * L * CW + lane, rows + ((size_t)TW + wv * L) * CW + lane,
                                        cok ? L : 0, wc, uc, ew, kmax, fast, Xs);
    sF[(0 * S + wv) * CW + lane] = sum.a;
    sF[(1 * S + wv) * CW + lane] = sum.b;
    sF[(2 * S + wv) * CW + lane] = sum.k;
    sF[(3 * S + wv) * CW + lane] = sum.n;
    __syncthreads();
    if (wv == 0) {
        St agg = st_empty();
        for (int j = 0; j < S; ++j) {
            const St sj = St{sF[(0 * S + j) * CW + lane], sF[(1 * S + j) * CW + lane],
                             sF[(2 * S + j) * CW + lane], sF[(3 * S + j) * CW + lane]};
            agg = (j == 0) ? sj : combine(agg, sj, (float)L, wc);
        }
        const int64_t chain = (b * nCT + ct) * nTT;
        f4 out;
        out[0] = agg.a;
        out[1] = agg.b;
        out[2] = agg.k;
        out[3] = agg.n;
        reinterpret_cast<f4 *>(ws.aggs)[(chain + tt) * CW + lane] = out;
    }
}

template <typename TIn>
__global__ void __launch_bounds__(256) wkv_passthrough_kernel(ForwardArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t BC = a.B * a.C;
    if (i >= BC) return;
    if (a.state_out) {
        if (a.state_in) {
            const float sa = a.state_in[i], sb = a.state_in[BC + i], sp = a.state_in[2 * BC + i];
            a.state_out[i] = sa;
            a.state_out[BC + i] = sb;
            a.state_out[2 * BC + i] = sp;
        } else {
            a.state_out[i] = 0.f;
            a.state_out[BC + i] = 0.f;
            a.state_out[2 * BC + i] = kEmptyP;
        }
    }
    if (a.mode == MODE_TIMEMIX && a.x_last) {
        const TIn *XP = static_cast<const TIn *>(a.x_prev);
        static_cast<TIn *>(a.x_last)[i] = XP ? XP[i] : (TIn)0;
    }
}

// Workgroups of a kernel the current device holds at once (occupancy x compute units), per
// kernel, launch shape and device, computed once; 0 when the runtime cannot say.
int64_t resident_slots(const void *kernel, int threads, size_t lds) {
    constexpr int kMaxDevices = 64;
    struct Entry {
        const void *kernel;
        int threads;
        size_t lds;
        int64_t slots;
    };
    static std::mutex mu;
    static std::vector<Entry> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry &e : cache[dev])
        if (e.kernel == kernel && e.threads == threads && e.lds == lds) return e.slots;
    int per_cu = 0, cus = 0;
    int64_t slots = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        slots = (int64_t)per_cu * cus;
    (void)hipGetLastError();  // a failed query leaves no sticky error behind
    cache[dev].push_back(Entry{kernel, threads, lds, slots});
    return slots;
}

template <typename TIn, typename TOut, int MODE>
hipError_t launch_seq_t(const ForwardArgs &a, hipStream_t s) {
    const int64_t threads = a.B * ((a.C + 3) / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((wkv_seq_kernel<TIn, TOut, MODE>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut, int MODE, int L, int PREFIX>
hipError_t launch_tile(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    const int S = chunk_len / L;
    const int nCT = (int)((a.C + kTileChannels - 1) / kTileChannels);
    const int nTT = (int)((a.T + chunk_len - 1) / chunk_len);
    const int64_t blocks = a.B * (int64_t)nCT * nTT;
    constexpr int NT = (MODE == MODE_PLAIN) ? 2 : 3;
    // staged rows + wave summaries (later the parts of the incoming state).  28 KB for the
    // fp16 time-mix at 64 tokens: LDS is allocated in granules that make 32 KB fit only 4
    // workgroups per CU (160 KB), 28 KB five.
    const size_t lds = (size_t)NT * chunk_len * kTileChannels * sizeof(TIn) + (size_t)4 * S * kTileChannels * sizeof(float);
    if (lds > kTileLdsMax) return hipErrorInvalidConfiguration;
    if (blocks > 0x7fffffff || S < 1 || 64 * S > 1024) return hipErrorInvalidConfiguration;
    constexpr bool kWide = L == 32 && MODE == MODE_PLAIN;  // 16-wave tiles of 32-token waves
    // each kernel's launch bounds: 8-token waves up to 4 per workgroup, 32-token waves up to 8
    // (16 ungated), 16-token waves up to 16
    if ((L == 8 && S > 4) || (L == 32 && S > (kWide ? 16 : 8))) return hipErrorInvalidConfiguration;
    if (PREFIX == PREFIX_AGGS && nTT > 1) {
        // first pass: aggregates of the first nTT - 1 time tiles (k and v rows only)
        const int64_t agg_blocks = a.B * (int64_t)nCT * (nTT - 1);
        const size_t lds1 = (size_t)2 * chunk_len * kTileChannels * sizeof(TIn) +
                            (size_t)4 * S * kTileChannels * sizeof(float);
        hipLaunchKernelGGL((wkv_tile_agg_kernel<TIn, L>), dim3((unsigned)agg_blocks), dim3(64 * S), lds1, s, a, ws,
                           S, nCT, nTT, chunk_len);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const void *kern;  // only the kernels for L are instantiated
    if constexpr (L == 32)
        kern = reinterpret_cast<const void *>(&wkv_tile32_kernel<TIn, TOut, MODE, PREFIX>);
    else if constexpr (L == 8)
        kern = reinterpret_cast<const void *>(&wkv_tile8_kernel<TIn, TOut, MODE, PREFIX>);
    else
        kern = reinterpret_cast<const void *>(&wkv_tile_kernel<TIn, TOut, MODE, PREFIX>);
    if constexpr (kWide)
        if (S > 8) kern = reinterpret_cast<const void *>(&wkv_tile32w_kernel<TIn, TOut, MODE, PREFIX>);
    const int64_t slots = resident_slots(kern, 64 * S, lds);
    // States go into the publishing XCD's L2 first when every tile of a chain runs on one XCD:
    // workgroup i runs on XCD i mod 8, tile (tt, chain r) is workgroup tt * G + r with G
    // workgroups per time tile, so without the per-tile rotation that holds when G is a
    // multiple of 8.  G is B * nCT, padded to a multiple of 8 with workgroups that return at
    // once when the padded grid still fits in one round and adds at most half again.
    const int64_t BCT = a.B * (int64_t)nCT, Gp = (BCT + 7) / 8 * 8;
    const bool pad = PREFIX == PREFIX_LOOKBACK && nTT > 1 && a.publish != RWKV_PUBLISH_WRITE_THROUGH &&
                     Gp != BCT && slots > 0 && Gp * nTT <= slots && 2 * Gp <= 3 * BCT;
    const int64_t G = pad ? Gp : BCT;
    const int64_t grid = G * nTT;
    const int rot = (slots > 0 && grid > slots) ? 1 : 0;  // more than one round of workgroups
    // Anchor spacing.  Within one round every tile is in flight at once and an anchor every 16
    // tiles leaves a chain of up to 16 tiles with no serial anchor hop.  Past one round the tiles
    // of a chain arrive in order; for 128-token tiles an anchor every 8 halves the words each
    // look-back reads (B1 T65536 C2048: 238.8 -> 234.9 us; every 4: 273 us, the anchors' own
    // chain too slow), while 64-token tiles, twice as many per chain, keep 16 (308 -> 324 us at 8).
    // Each wave of a look-back folds at most kMaxAnchorGap / 4 tiles, so a workgroup of fewer
    // than 4 waves (16-token tiles) anchors every 4 S tiles.
    const int M = std::min((rot && L == 32) ? kMaxAnchorGap / 2 : kMaxAnchorGap, 4 * S);
    const bool one_xcd = rot == 0 && G % 8 == 0;
    const int lp = PREFIX == PREFIX_LOOKBACK && (a.publish == RWKV_PUBLISH_L2_FIRST ||
                                                 (a.publish == RWKV_PUBLISH_AUTO && one_xcd));
    if constexpr (kWide) {
        if (S > 8) {
            hipLaunchKernelGGL((wkv_tile32w_kernel<TIn, TOut, MODE, PREFIX>), dim3((unsigned)grid), dim3(64 * S), lds,
                               s, a, ws, S, nCT, nTT, chunk_len, M, rot, lp, (int)G);
            return hipGetLastError();
        }
    }
    if constexpr (L == 32)
        hipLaunchKernelGGL((wkv_tile32_kernel<TIn, TOut, MODE, PREFIX>), dim3((unsigned)grid), dim3(64 * S), lds, s,
                           a, ws, S, nCT, nTT, chunk_len, M, rot, lp, (int)G);
    else if constexpr (L == 8)
        hipLaunchKernelGGL((wkv_tile8_kernel<TIn, TOut, MODE, PREFIX>), dim3((unsigned)grid), dim3(64 * S), lds, s,
                           a, ws, S, nCT, nTT, chunk_len, M, rot, lp, (int)G);
    else
        hipLaunchKernelGGL((wkv_tile_kernel<TIn, TOut, MODE, PREFIX>), dim3((unsigned)grid), dim3(64 * S), lds, s,
                           a, ws, S, nCT, nTT, chunk_len, M, rot, lp, (int)G);
    return hipGetLastError();
}

// Long tiles: chunk_len / (4 L) sub-tiles of 4 waves x L tokens, L = 32 for 2-byte inputs and
// 16 for fp32 (the staged tile lengths of launch_tile).
template <typename TIn, typename TOut, int MODE, int L>
hipError_t launch_long(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    constexpr int S = 4;
    constexpr int NT = (MODE == MODE_PLAIN) ? 2 : 3;
    const int nCT = (int)((a.C + kTileChannels - 1) / kTileChannels);
    const int64_t nTT = (a.T + chunk_len - 1) / chunk_len;
    const int64_t BCT = a.B * (int64_t)nCT;
    const int64_t grid = BCT * nTT;
    if (grid > 0x7fffffff || chunk_len % (S * L) != 0 || BCT > 0x7fffffff) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)NT * S * L * kTileChannels * sizeof(TIn) + (size_t)4 * S * kTileChannels * sizeof(float);
    const void *kern;  // only the kernel for L is instantiated
    if constexpr (L == 32)
        kern = reinterpret_cast<const void *>(&wkv_long32_kernel<TIn, TOut, MODE>);
    else
        kern = reinterpret_cast<const void *>(&wkv_long16_kernel<TIn, TOut, MODE>);
    const int64_t slots = resident_slots(kern, 64 * S, lds);
    const int rot = (slots > 0 && grid > slots) ? 1 : 0;
    if constexpr (L == 32)
        hipLaunchKernelGGL((wkv_long32_kernel<TIn, TOut, MODE>), dim3((unsigned)grid), dim3(64 * S), lds, s, a, ws, S,
                           nCT, (int)nTT, chunk_len, kMaxAnchorGap, rot, (int)BCT);
    else
        hipLaunchKernelGGL((wkv_long16_kernel<TIn, TOut, MODE>), dim3((unsigned)grid), dim3(64 * S), lds, s, a, ws, S,
                           nCT, (int)nTT, chunk_len, kMaxAnchorGap, rot, (int)BCT);
    return hipGetLastError();
}

// 16- and 32-token tiles: 2 or 4 waves of 8 tokens; 64-token tiles: 4 waves of 16 tokens;
// longer tiles: waves of 32 tokens (2-byte inputs) or 16 (fp32), 4 to 16 of them, as long as
// the tile's rows fit in LDS (ungated: 512 tokens of 2-byte rows, 256 of fp32; gated and time
// mix: 256 and 128); longer chunks (up to kMaxChunk) as long tiles of 4-wave sub-tiles.
// Measured on one MI355X, a staged tile beats the long tile of the same length, which reads
// k and v twice: B1 T65536 C2048 fp16 -> fp32 at 256 tokens 233 against 332 us, at 512 268
// against 321 us; the 14B time mix at 256 tokens 19.5 against 24.9 us.
template <typename TIn, typename TOut, int MODE>
hipError_t launch_chunk_t(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    if (chunk_len <= 32) return launch_tile<TIn, TOut, MODE, 8, PREFIX_LOOKBACK>(a, chunk_len, ws, s);
    constexpr int L = sizeof(TIn) == 2 ? 32 : 16;
    if (chunk_len > staged_tile_max<TIn, MODE>()) return launch_long<TIn, TOut, MODE, L>(a, chunk_len, ws, s);
    if (chunk_len >= 4 * L) return launch_tile<TIn, TOut, MODE, L, PREFIX_LOOKBACK>(a, chunk_len, ws, s);
    return launch_tile<TIn, TOut, MODE, 16, PREFIX_LOOKBACK>(a, chunk_len, ws, s);
}

// The two-pass scan stages every tile whole (chunk_len up to staged_tile_max, checked by the
// caller), in the same tile shapes as the single pass.
template <typename TIn, typename TOut, int MODE>
hipError_t launch_chunk2_t(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    if (chunk_len <= 32) return launch_tile<TIn, TOut, MODE, 8, PREFIX_AGGS>(a, chunk_len, ws, s);
    constexpr int L = sizeof(TIn) == 2 ? 32 : 16;
    if (chunk_len > staged_tile_max<TIn, MODE>()) return hipErrorInvalidValue;
    if (chunk_len >= 4 * L) return launch_tile<TIn, TOut, MODE, L, PREFIX_AGGS>(a, chunk_len, ws, s);
    return launch_tile<TIn, TOut, MODE, 16, PREFIX_AGGS>(a, chunk_len, ws, s);
}

// This translation unit instantiates the kernels of one input dtype, RWKV_TU_IN (rwkv_dtype
// code: 0 fp32, 1 fp16, 2 bf16); the build compiles the file once per input dtype, in parallel.
#if RWKV_TU_IN == 0
using TuIn = float;
#elif RWKV_TU_IN == 1
using TuIn = _Float16;
#else
using TuIn = __bf16;
#endif

// Every (output dtype, mode) instantiation for this unit's input dtype.
#define RWKV_DISPATCH_MODE(LAUNCH, TO, ...)                                          \
    do {                                                                             \
        if (a.mode == MODE_PLAIN) return LAUNCH<TuIn, TO, MODE_PLAIN>(__VA_ARGS__); \
        if (a.mode == MODE_GATED) return LAUNCH<TuIn, TO, MODE_GATED>(__VA_ARGS__); \
        return LAUNCH<TuIn, TO, MODE_TIMEMIX>(__VA_ARGS__);                          \
    } while (0)
#define RWKV_DISPATCH(LAUNCH, ...)                                                   \
    do {                                                                             \
        if (a.out_dt == 1) RWKV_DISPATCH_MODE(LAUNCH, _Float16, __VA_ARGS__);        \
        if (a.out_dt == 2) RWKV_DISPATCH_MODE(LAUNCH, __bf16, __VA_ARGS__);          \
        RWKV_DISPATCH_MODE(LAUNCH, float, __VA_ARGS__);                              \
    } while (0)

}  // namespace

#define RWKV_TU_NAME2(f, k) f##_in##k
#define RWKV_TU_NAME1(f, k) RWKV_TU_NAME2(f, k)
#define RWKV_TU_NAME(f) RWKV_TU_NAME1(f, RWKV_TU_IN)

hipError_t RWKV_TU_NAME(launch_sequential)(const ForwardArgs &a, hipStream_t s) { RWKV_DISPATCH(launch_seq_t, a, s); }

hipError_t RWKV_TU_NAME(launch_chunked)(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    RWKV_DISPATCH(launch_chunk_t, a, chunk_len, ws, s);
}

hipError_t RWKV_TU_NAME(launch_chunked_2pass)(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws,
                                             hipStream_t s) {
    RWKV_DISPATCH(launch_chunk2_t, a, chunk_len, ws, s);
}

#if RWKV_TU_IN == 0
// Longest tile staged in LDS at once (the two-pass scan's limit; the single-launch scan runs
// longer chunks as long tiles).
int tile_max_len(int in_2byte, int gated) {
    if (in_2byte)
        return gated ? staged_tile_max<_Float16, MODE_GATED>() : staged_tile_max<_Float16, MODE_PLAIN>();
    return gated ? staged_tile_max<float, MODE_GATED>() : staged_tile_max<float, MODE_PLAIN>();
}

bool auto_sequential(int64_t B, int64_t T, int64_t C) {
    // Enough independent (b, channel) lanes to fill every SIMD twice over: the
    // sequential kernel then reads each input once with no scan overhead.
    const int64_t lanes = B * ((C + 3) / 4);
    return lanes >= 131072 || T <= 1;
}

int auto_chunk_len(int64_t B, int64_t T, int64_t C, int in_2byte) {
    (void)B;
    (void)C;
    (void)T;
    // 2-byte inputs (fp16, bf16): 128-token tiles of 4 waves x 32 tokens.  Against 64-token tiles (4 x 16) they halve
    // the tiles per chain and quarter the look-back reads, and three 52 KB workgroups per CU
    // still hold a layer-sized call at once: 14B layer 18.2 -> 17.3 us, 169m batch 20.6 ->
    // 18.1 us, B1 T65536 C2048 386 -> 286 us.  fp32 rows are twice the size: 64 tokens.
    return in_2byte ? 128 : 64;
}

size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t C, int chunk_len) {
    const int64_t nCT = (C + kTileChannels - 1) / kTileChannels;
    const int64_t nTT = (T + chunk_len - 1) / chunk_len;
    const int64_t tiles = B * nCT * nTT;
    // a 256-byte header (the error word), then words [tiles][4][64] u64 (one published state
    // per tile, single pass), then aggregates [tiles][64][4] fp32 (two passes).  The two
    // regions are disjoint, so a float left by one algorithm can never pass for a tagged word.
    return (size_t)(256 + tiles * 4 * kTileChannels * 8 + tiles * kTileChannels * 4 * 4);
}

void chunk_workspace_carve(void *base, int64_t B, int64_t T, int64_t C, int chunk_len,
                           ChunkWorkspace *ws) {
    const int64_t nCT = (C + kTileChannels - 1) / kTileChannels;
    const int64_t nTT = (T + chunk_len - 1) / chunk_len;
    const int64_t tiles = B * nCT * nTT;
    char *p = static_cast<char *>(base);
    // The error word sits at a fixed place whatever the shape: it must read 0 unless a wait
    // gave up, and one workspace serves calls of different shapes, whose word regions
    // overwrite each other (a stale tagged word read as the error word would make every wait
    // longer than 64 polls give up at once).
    ws->err = reinterpret_cast<uint32_t *>(p);
    ws->words = reinterpret_cast<uint64_t *>(p + 256);
    ws->aggs = reinterpret_cast<float *>(p + 256 + tiles * 4 * kTileChannels * 8);
}

#define RWKV_BY_IN(F, ...) \
    (a.in_dt == 1 ? F##_in1(__VA_ARGS__) : a.in_dt == 2 ? F##_in2(__VA_ARGS__) : F##_in0(__VA_ARGS__))

hipError_t launch_sequential(const ForwardArgs &a, hipStream_t s) { return RWKV_BY_IN(launch_sequential, a, s); }

hipError_t launch_chunked(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    return RWKV_BY_IN(launch_chunked, a, chunk_len, ws, s);
}

hipError_t launch_chunked_2pass(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s) {
    return RWKV_BY_IN(launch_chunked_2pass, a, chunk_len, ws, s);
}

hipError_t launch_passthrough(const ForwardArgs &a, hipStream_t s) {
    const int64_t n = a.B * a.C;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (a.in_dt == 1)
        hipLaunchKernelGGL((wkv_passthrough_kernel<_Float16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else if (a.in_dt == 2)
        hipLaunchKernelGGL((wkv_passthrough_kernel<__bf16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((wkv_passthrough_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}
#endif  // RWKV_TU_IN == 0

}  // namespace rwkvwkv
