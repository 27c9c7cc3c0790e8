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
//   wkv_chunk_kernel  one workgroup per (b, 64 channels, tile of TW tokens); each lane
//                     keeps 16 tokens x 4 channels of k, v (and r or x) in VGPRs,
//                     reduces them to a summary, the workgroup scans the summaries in
//                     LDS, a decoupled look-back over earlier tiles supplies the
//                     incoming state, and each lane replays its tokens to emit y.
//                     HBM traffic is one read of each input and one write of y.
//   wkv_passthrough   T = 0: copy the state (and x_prev to x_last).

#include "wkv_internal.h"

#include <algorithm>

namespace rwkvwkv {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEmptyP = -1.0e38f;  // p of the empty state (finite, so differences stay defined)
constexpr uint32_t kAgg = 1u, kIncl = 2u;
constexpr uint32_t kMaxSpins = 1u << 20;  // ~25 ms of polling before a look-back gives up
constexpr int kMaxAnchorGap = 32;         // largest spacing of anchor tiles in a chain

template <typename T> struct Raw;
template <> struct Raw<float> { using type = f4; };
template <> struct Raw<_Float16> { using type = h4; };

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
template <typename T>
__device__ __forceinline__ typename Raw<T>::type load4(const T *p, int64_t off, int nch, bool vec) {
    using R = typename Raw<T>::type;
    R r = {0, 0, 0, 0};
    if (vec) {
        if (nch == 4) r = *reinterpret_cast<const R *>(p + off);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nch) r[q] = p[off + q];
    }
    return r;
}

template <typename T>
__device__ __forceinline__ void store4(T *p, int64_t off, int nch, bool vec, const float (&x)[4]) {
    using R = typename Raw<T>::type;
    if (vec) {
        if (nch == 4) {
            R r;
#pragma unroll
            for (int q = 0; q < 4; ++q) r[q] = (T)x[q];  // fp16: round to nearest even
            *reinterpret_cast<R *>(p + off) = r;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nch) p[off + q] = (T)x[q];
    }
}

__device__ __forceinline__ void load_param4(const float *p, int64_t c0, int nch, float (&x)[4]) {
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
    load_param4(a.w, c0, nch, w);
    load_param4(a.u, c0, nch, u);
    St s[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w[q] = finite_decay(w[q]);
        s[q] = st_empty();
        if (a.state_in && q < nch)
            s[q] = st_load(a.state_in[sc + q], a.state_in[BC + sc + q], a.state_in[2 * BC + sc + q]);
    }
    float mk[4], mv[4], mr[4], xs[4];
    if constexpr (MODE == MODE_TIMEMIX) {
        load_param4(a.mix_k, c0, nch, mk);
        load_param4(a.mix_v, c0, nch, mv);
        load_param4(a.mix_r, c0, nch, mr);
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
    if (a.state_out) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < nch) {
                a.state_out[sc + q] = s[q].a;
                a.state_out[BC + sc + q] = s[q].b;
                a.state_out[2 * BC + sc + q] = st_logmax(s[q], w[q]);
            }
    }
    if constexpr (MODE == MODE_TIMEMIX) {
        if (a.x_last) store4(static_cast<TIn *>(a.x_last), sc, nch, vec, xs);
    }
}

// ------------------------------------------------------------------------------------------
// Chunked scan.

__device__ __forceinline__ void publish(const ChunkWorkspace &ws, int64_t tile, uint32_t kind,
                                        const St &s, int ch) {
    uint32_t *dst = reinterpret_cast<uint32_t *>(kind == kIncl ? ws.incl : ws.agg) + tile * (4 * kTileChannels);
    const float f[4] = {s.a, s.b, s.k, s.n};
#pragma unroll
    for (int m = 0; m < 4; ++m)
        __hip_atomic_store(dst + m * kTileChannels + ch, __float_as_uint(f[m]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    // release: this lane's data before this lane's flag (one flag word per channel)
    __hip_atomic_store(ws.flags + tile * kTileChannels + ch, (ws.epoch << 2) | kind,
                       __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Incoming state of tile tt >= 1 of a chain.  Anchor tiles (every M-th, tile 0 included)
// publish their inclusive state; the others publish only their own aggregate.  With a the
// last anchor before tt, the prefix is INCL(a) + AGG(a+1) + ... + AGG(tt-1), folded in that
// fixed order whatever the timing, so results are bitwise reproducible.  All the flags are
// polled together: one round trip, not one per tile.
__device__ St lookback(const ChunkWorkspace &ws, int64_t chain, int64_t tt, float wc, int TW, int M,
                       int ch) {
    const int64_t a = ((tt - 1) / M) * M;
    const int cnt = (int)(tt - a);  // tiles a .. tt-1, 1 <= cnt <= M <= kMaxAnchorGap
    uint32_t spins = 0;
    for (;;) {
        bool all = true;
#pragma unroll
        for (int m = 0; m < kMaxAnchorGap; ++m) {
            if (m < cnt) {
                const uint32_t f = __hip_atomic_load(ws.flags + (chain + a + m) * kTileChannels + ch,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                all = all && (f >> 2) == ws.epoch;
            }
        }
        if (all) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            break;
        }
        ++spins;
        // give up after kMaxSpins, or at once when another wait has already given up
        if (spins > kMaxSpins ||
            ((spins & 255u) == 0 && __hip_atomic_load(ws.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
            atomicOr(ws.err, 1u);
            return St{__builtin_nanf(""), __builtin_nanf(""), 0.f, 0.f};  // poison the tile's outputs
        }
        __builtin_amdgcn_s_sleep(1);
    }
    St acc = st_empty();
    float acc_len = 0.f;
#pragma unroll
    for (int m = kMaxAnchorGap - 1; m >= 0; --m) {
        if (m < cnt) {
            const int64_t tile = chain + a + m;
            const uint32_t *src =
                reinterpret_cast<const uint32_t *>(m == 0 ? ws.incl : ws.agg) + tile * (4 * kTileChannels);
            float x[4];
#pragma unroll
            for (int f = 0; f < 4; ++f)
                x[f] = __uint_as_float(
                    __hip_atomic_load(src + f * kTileChannels + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            acc = combine(St{x[0], x[1], x[2], x[3]}, acc, acc_len, wc);
            acc_len += (float)TW;
        }
    }
    return acc;
}

template <typename TIn, int MODE>
constexpr int chunk_max_threads() {
    return (sizeof(TIn) == 2 && MODE == MODE_PLAIN) ? 1024 : 512;
}

// Workgroup = (b, channel tile ct of 64 channels, time tile tt of TW = 16*S tokens),
// blockIdx = tt * (B * nCT) + b * nCT + ct, so every tile a workgroup waits for has a
// lower index and was dispatched earlier.  Thread = (sub-chunk j, channel group g):
// tid = j * 16 + g, channels ct*64 + 4g .. +3, tokens tt*TW + 16j .. +15.
// LDS: per sub-chunk and channel the four fields of a state, then the tile's incoming state.
template <typename TIn, typename TOut, int MODE>
__global__ void __launch_bounds__((chunk_max_threads<TIn, MODE>()))
    wkv_chunk_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW, int M) {
    constexpr int L = kSubLen, G = 16, CW = kTileChannels;
    using R = typename Raw<TIn>::type;
    extern __shared__ float smem[];
    float *sF[4] = {smem, smem + S * CW, smem + 2 * S * CW, smem + 3 * S * CW};
    float *sI = smem + 4 * S * CW;  // [4][CW]

    const int tid = threadIdx.x, g = tid % G, j = tid / G;
    const int64_t BCT = a.B * nCT;
    const int64_t tt = blockIdx.x / BCT;
    const int64_t rem = blockIdx.x - tt * BCT;
    const int64_t b = rem / nCT, ct = rem - b * nCT;
    const int64_t c0 = ct * CW + g * 4;
    const int nch = (int)std::max<int64_t>(0, std::min<int64_t>(4, a.C - c0));
    const int64_t tile_t0 = tt * TW;
    const int64_t tile_len = std::min<int64_t>(TW, a.T - tile_t0);
    const int64_t t0 = tile_t0 + (int64_t)j * L;
    const int nval = (int)std::max<int64_t>(0, std::min<int64_t>(L, a.T - t0));
    const bool vec = a.vec != 0;
    const int64_t BC = a.B * a.C, sc = b * a.C + c0;

    const TIn *K = static_cast<const TIn *>(a.k);
    const TIn *V = static_cast<const TIn *>(a.v);
    const TIn *GR = static_cast<const TIn *>(MODE == MODE_GATED ? a.r : a.x);

    float w[4], u[4];
    load_param4(a.w, c0, nch, w);
    load_param4(a.u, c0, nch, u);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = finite_decay(w[q]);

    // Phase A: every load of the lane's tile slice is issued up front.
    const int64_t base = (b * a.T + t0) * a.C + c0;
    R kr[L], vr[L], gr[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = i < nval;
        kr[i] = ok ? load4(K, base + i * a.C, nch, vec) : R{0, 0, 0, 0};
        vr[i] = ok ? load4(V, base + i * a.C, nch, vec) : R{0, 0, 0, 0};
        if constexpr (MODE != MODE_PLAIN) gr[i] = ok ? load4(GR, base + i * a.C, nch, vec) : R{0, 0, 0, 0};
    }
    R xp = {0, 0, 0, 0};
    float mk[4], mv[4], mr[4];
    if constexpr (MODE == MODE_TIMEMIX) {
        load_param4(a.mix_k, c0, nch, mk);
        load_param4(a.mix_v, c0, nch, mv);
        load_param4(a.mix_r, c0, nch, mr);
        if (nval > 0) {
            if (t0 > 0)
                xp = load4(GR, base - a.C, nch, vec);
            else if (a.x_prev)
                xp = load4(static_cast<const TIn *>(a.x_prev), sc, nch, vec);
        }
    }

    // Phase B: summary of the lane's sub-chunk from the empty state.
    St sum[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] = st_empty();
#pragma unroll
    for (int i = 0; i < L; ++i) {
        if (i < nval) {
#pragma unroll
            for (int q = 0; q < 4; ++q) absorb(sum[q], w[q], (float)kr[i][q], (float)vr[i][q]);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = j * CW + g * 4 + q;
        sF[0][idx] = sum[q].a;
        sF[1][idx] = sum[q].b;
        sF[2][idx] = sum[q].k;
        sF[3][idx] = sum[q].n;
    }
    __syncthreads();

    // Phase C: one lane per channel scans the S summaries (exclusive, from the tile start),
    // then fetches the tile's incoming state.
    if (tid < CW) {
        const int ch = tid;
        const int64_t c = ct * CW + ch;
        const bool cok = c < a.C;
        const float wc = cok ? finite_decay(a.w[c]) : 0.f;
        St run = st_empty();
        float run_len = 0.f;
        for (int jj = 0; jj < S; ++jj) {
            const int64_t len = std::max<int64_t>(0, std::min<int64_t>(L, a.T - (tile_t0 + (int64_t)jj * L)));
            const int idx = jj * CW + ch;
            const St cur = St{sF[0][idx], sF[1][idx], sF[2][idx], sF[3][idx]};
            sF[0][idx] = run.a;
            sF[1][idx] = run.b;
            sF[2][idx] = run.k;
            sF[3][idx] = run.n;
            run = combine(run, cur, (float)len, wc);
            run_len += (float)len;
        }
        St prefix = st_empty();
        if (tt == 0 && a.state_in && cok) {
            const int64_t s = b * a.C + c;
            prefix = st_load(a.state_in[s], a.state_in[BC + s], a.state_in[2 * BC + s]);
        }
        if (nTT > 1) {
            const int64_t chain = (b * nCT + ct) * nTT;
            const bool anchor = (tt % M) == 0, last = tt == nTT - 1;
            if (!anchor && !last) publish(ws, chain + tt, kAgg, run, ch);
            if (tt > 0) prefix = lookback(ws, chain, tt, wc, TW, M, ch);
            if (anchor && !last) publish(ws, chain + tt, kIncl, combine(prefix, run, run_len, wc), ch);
        }
        sI[ch] = prefix.a;
        sI[CW + ch] = prefix.b;
        sI[2 * CW + ch] = prefix.k;
        sI[3 * CW + ch] = prefix.n;
    }
    __syncthreads();

    // Phase D: the lane's starting state = tile prefix, then the sub-chunks before it.
    St st[4];
    const float before = (float)std::min<int64_t>((int64_t)j * L, tile_len);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cl = g * 4 + q, jl = j * CW + cl;
        const St pre = St{sI[cl], sI[CW + cl], sI[2 * CW + cl], sI[3 * CW + cl]};
        const St exl = St{sF[0][jl], sF[1][jl], sF[2][jl], sF[3][jl]};
        st[q] = combine(pre, exl, before, w[q]);
    }

    // Phase E: replay the tokens from registers, emit y.
    TOut *Y = static_cast<TOut *>(a.y);
    float xs[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xs[q] = (float)xp[q];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        if (i < nval) {
            float yv[4], xko[4], xvo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float kk = (float)kr[i][q], vv = (float)vr[i][q];
                float num, den;
                emit(st[q], w[q], u[q], kk, vv, num, den);
                float gt = 1.f;
                if constexpr (MODE == MODE_GATED) gt = 1.f + ex(-(float)gr[i][q]);
                if constexpr (MODE == MODE_TIMEMIX) {
                    const float xx = (float)gr[i][q];
                    const float xr = mr[q] * xx + (1.f - mr[q]) * xs[q];
                    xko[q] = mk[q] * xx + (1.f - mk[q]) * xs[q];
                    xvo[q] = mv[q] * xx + (1.f - mv[q]) * xs[q];
                    xs[q] = xx;
                    gt = 1.f + ex(-xr);
                }
                yv[q] = num * rcp(den * gt);
                absorb(st[q], w[q], kk, vv);
            }
            const int64_t off = base + i * a.C;
            store4(Y, off, nch, vec, yv);
            if constexpr (MODE == MODE_TIMEMIX) {
                if (a.xk_out) store4(static_cast<TIn *>(a.xk_out), off, nch, vec, xko);
                if (a.xv_out) store4(static_cast<TIn *>(a.xv_out), off, nch, vec, xvo);
            }
        }
    }

    // Phase F: the lane holding token T-1 writes the final state (and x_last).
    if (nval > 0 && t0 + nval == a.T) {
        if (a.state_out) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < nch) {
                    a.state_out[sc + q] = st[q].a;
                    a.state_out[BC + sc + q] = st[q].b;
                    a.state_out[2 * BC + sc + q] = st_logmax(st[q], w[q]);
                }
        }
        if constexpr (MODE == MODE_TIMEMIX) {
            if (a.x_last) store4(static_cast<TIn *>(a.x_last), sc, nch, vec, xs);
        }
    }
}

// ------------------------------------------------------------------------------------------

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

template <typename TIn, typename TOut, int MODE>
hipError_t launch_seq_t(const ForwardArgs &a, hipStream_t s) {
    const int64_t threads = a.B * ((a.C + 3) / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((wkv_seq_kernel<TIn, TOut, MODE>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut, int MODE>
hipError_t launch_chunk_t(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws,
                          hipStream_t s) {
    const int S = chunk_len / kSubLen;
    const int nCT = (int)((a.C + kTileChannels - 1) / kTileChannels);
    const int nTT = (int)((a.T + chunk_len - 1) / chunk_len);
    const int64_t blocks = a.B * (int64_t)nCT * nTT;
    const size_t lds = (size_t)(4 * S * kTileChannels + 4 * kTileChannels) * sizeof(float);
    if (blocks > 0x7fffffff || 16 * S > chunk_max_threads<TIn, MODE>()) return hipErrorInvalidConfiguration;
    // anchor spacing ~ sqrt(tiles per chain): the anchor chain and each tile's fold stay short
    int M = 4;
    while (M < kMaxAnchorGap && (int64_t)M * M < nTT) M <<= 1;
    hipLaunchKernelGGL((wkv_chunk_kernel<TIn, TOut, MODE>), dim3((unsigned)blocks), dim3(16 * S), lds,
                       s, a, ws, S, nCT, nTT, chunk_len, M);
    return hipGetLastError();
}

#define RWKV_DISPATCH(LAUNCH, ...)                                                              \
    do {                                                                                        \
        if (a.in_f16) {                                                                         \
            if (a.out_f16) {                                                                    \
                if (a.mode == MODE_PLAIN) return LAUNCH<_Float16, _Float16, MODE_PLAIN>(__VA_ARGS__); \
                if (a.mode == MODE_GATED) return LAUNCH<_Float16, _Float16, MODE_GATED>(__VA_ARGS__); \
                return LAUNCH<_Float16, _Float16, MODE_TIMEMIX>(__VA_ARGS__);                   \
            }                                                                                   \
            if (a.mode == MODE_PLAIN) return LAUNCH<_Float16, float, MODE_PLAIN>(__VA_ARGS__);  \
            if (a.mode == MODE_GATED) return LAUNCH<_Float16, float, MODE_GATED>(__VA_ARGS__);  \
            return LAUNCH<_Float16, float, MODE_TIMEMIX>(__VA_ARGS__);                          \
        }                                                                                       \
        if (a.out_f16) {                                                                        \
            if (a.mode == MODE_PLAIN) return LAUNCH<float, _Float16, MODE_PLAIN>(__VA_ARGS__);  \
            if (a.mode == MODE_GATED) return LAUNCH<float, _Float16, MODE_GATED>(__VA_ARGS__);  \
            return LAUNCH<float, _Float16, MODE_TIMEMIX>(__VA_ARGS__);                          \
        }                                                                                       \
        if (a.mode == MODE_PLAIN) return LAUNCH<float, float, MODE_PLAIN>(__VA_ARGS__);         \
        if (a.mode == MODE_GATED) return LAUNCH<float, float, MODE_GATED>(__VA_ARGS__);         \
        return LAUNCH<float, float, MODE_TIMEMIX>(__VA_ARGS__);                                 \
    } while (0)

}  // namespace

int chunk_max_len(int in_f16, int mode) { return (in_f16 && mode == MODE_PLAIN) ? 1024 : 512; }

bool auto_sequential(int64_t B, int64_t T, int64_t C) {
    // Enough independent (b, channel) lanes to fill every SIMD twice over: the
    // sequential kernel then reads each input once with no scan overhead.
    const int64_t lanes = B * ((C + 3) / 4);
    return lanes >= 131072 || T <= 1;
}

int auto_chunk_len(int64_t B, int64_t T, int64_t C) {
    (void)B;
    (void)C;
    int len = kMinChunk;
    while (len < 256 && (int64_t)len * 4 < T) len <<= 1;
    return len;
}

size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t C, int chunk_len) {
    const int64_t nCT = (C + kTileChannels - 1) / kTileChannels;
    const int64_t nTT = (T + chunk_len - 1) / chunk_len;
    const int64_t tiles = B * nCT * nTT;
    // flags [tiles][64] u32 + agg, incl [tiles][4][64] f32 + one error word, 256-B aligned parts
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    return (size_t)(al(tiles * kTileChannels * 4) + 2 * al(tiles * 4 * kTileChannels * 4) + 256);
}

void chunk_workspace_carve(void *base, int64_t B, int64_t T, int64_t C, int chunk_len,
                           ChunkWorkspace *ws) {
    const int64_t nCT = (C + kTileChannels - 1) / kTileChannels;
    const int64_t nTT = (T + chunk_len - 1) / chunk_len;
    const int64_t tiles = B * nCT * nTT;
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    char *p = static_cast<char *>(base);
    ws->flags = reinterpret_cast<uint32_t *>(p);
    p += al(tiles * kTileChannels * 4);
    ws->agg = reinterpret_cast<float *>(p);
    p += al(tiles * 4 * kTileChannels * 4);
    ws->incl = reinterpret_cast<float *>(p);
    p += al(tiles * 4 * kTileChannels * 4);
    ws->err = reinterpret_cast<uint32_t *>(p);
}

hipError_t launch_sequential(const ForwardArgs &a, hipStream_t s) { RWKV_DISPATCH(launch_seq_t, a, s); }

hipError_t launch_chunked(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws,
                          hipStream_t s) {
    RWKV_DISPATCH(launch_chunk_t, a, chunk_len, ws, s);
}

hipError_t launch_passthrough(const ForwardArgs &a, hipStream_t s) {
    const int64_t n = a.B * a.C;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (a.in_f16)
        hipLaunchKernelGGL((wkv_passthrough_kernel<_Float16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((wkv_passthrough_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rwkvwkv
