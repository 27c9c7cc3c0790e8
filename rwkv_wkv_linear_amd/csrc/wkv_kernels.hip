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
// Spans compose: the state after a span of n tokens, started from (a1, b1, p1),
// is (a1, b1, p1 + n w) merged with the span's own summary from the empty state,
// by the same max rule.  This operator is associative, which the chunked scan
// uses to split T across lanes and workgroups.
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

template <typename T> struct Raw;
template <> struct Raw<float> { using type = f4; };
template <> struct Raw<_Float16> { using type = h4; };

__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

struct St {
    float a, b, p;
};

__device__ __forceinline__ St st_empty() { return St{0.f, 0.f, kEmptyP}; }

// Decay exponent of n tokens (0 when n == 0, also for w = -inf).
__device__ __forceinline__ float span_decay(int64_t n, float w) { return n ? (float)n * w : 0.f; }

// State s, then a span whose own summary (from the empty state) is t; dec = n * w.
__device__ __forceinline__ St combine(St s, St t, float dec) {
    const float P = s.p + dec;
    const float d = P - t.p;
    const float e = ex(-fabsf(d));
    const bool left = d >= 0.f;
    const float e1 = left ? 1.f : e, e2 = left ? e : 1.f;
    return St{s.a * e1 + t.a * e2, s.b * e1 + t.b * e2, left ? P : t.p};
}

// Absorb token (k, v).
__device__ __forceinline__ void absorb(St &s, float w, float k, float v) {
    const float pw = s.p + w;
    const float d = pw - k;
    const float e = ex(-fabsf(d));
    const bool left = d >= 0.f;
    const float e1 = left ? 1.f : e, e2 = left ? e : 1.f;
    s.a = s.a * e1 + v * e2;
    s.b = s.b * e1 + e2;
    s.p = left ? pw : k;
}

// Numerator and denominator of the output at token (k, v) with bonus u.
__device__ __forceinline__ void emit(const St &s, float u, float k, float v, float &num,
                                     float &den) {
    const float ku = u + k;
    const float d = s.p - ku;
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
        s[q] = st_empty();
        if (a.state_in && q < nch)
            s[q] = St{a.state_in[sc + q], a.state_in[BC + sc + q], a.state_in[2 * BC + sc + q]};
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
            emit(s[q], u[q], kk, vv, num, den);
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
                a.state_out[2 * BC + sc + q] = s[q].p;
            }
    }
    if constexpr (MODE == MODE_TIMEMIX) {
        if (a.x_last) store4(static_cast<TIn *>(a.x_last), sc, nch, vec, xs);
    }
}

// ------------------------------------------------------------------------------------------
// Chunked scan.

__device__ __forceinline__ void publish(const ChunkWorkspace &ws, int64_t tile, uint32_t kind,
                                        St s, int ch) {
    float *dst = (kind == kIncl ? ws.incl : ws.agg) + tile * (3 * kTileChannels);
    __hip_atomic_store(reinterpret_cast<uint32_t *>(dst) + ch, __float_as_uint(s.a),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint32_t *>(dst) + kTileChannels + ch, __float_as_uint(s.b),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint32_t *>(dst) + 2 * kTileChannels + ch,
                       __float_as_uint(s.p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // release: this lane's data before this lane's flag (one flag word per channel)
    __hip_atomic_store(ws.flags + tile * kTileChannels + ch, (ws.epoch << 2) | kind,
                       __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Incoming state of tile tt of a chain: walk back over earlier tiles, folding their
// aggregates, until one has published its inclusive state.
__device__ St lookback(const ChunkWorkspace &ws, int64_t chain, int64_t tt, float wc, int TW,
                       int ch) {
    St acc = st_empty();
    int64_t acc_len = 0;
    for (int64_t kk = tt - 1; kk >= 0; --kk) {
        const int64_t tile = chain + kk;
        uint32_t f = 0, spins = 0;
        for (;;) {
            f = __hip_atomic_load(ws.flags + tile * kTileChannels + ch, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            if ((f >> 2) == ws.epoch) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                break;
            }
            ++spins;
            // give up after kMaxSpins, or at once when another wait has already given up
            if (spins > kMaxSpins ||
                ((spins & 255u) == 0 &&
                 __hip_atomic_load(ws.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
                atomicOr(ws.err, 1u);
                f = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const uint32_t kind = f & 3u;
        if (kind == 0) {  // gave up: poison the tile so the failure shows in its outputs
            acc = St{__builtin_nanf(""), __builtin_nanf(""), 0.f};
            break;
        }
        const uint32_t *src =
            reinterpret_cast<const uint32_t *>(kind == kIncl ? ws.incl : ws.agg) + tile * (3 * kTileChannels);
        St x;
        x.a = __uint_as_float(__hip_atomic_load(src + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        x.b = __uint_as_float(
            __hip_atomic_load(src + kTileChannels + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        x.p = __uint_as_float(
            __hip_atomic_load(src + 2 * kTileChannels + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        acc = combine(x, acc, span_decay(acc_len, wc));
        acc_len += TW;
        if (kind == kIncl) break;
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
template <typename TIn, typename TOut, int MODE>
__global__ void __launch_bounds__((chunk_max_threads<TIn, MODE>()))
    wkv_chunk_kernel(ForwardArgs a, ChunkWorkspace ws, int S, int nCT, int nTT, int TW) {
    constexpr int L = kSubLen, G = 16, CW = kTileChannels;
    using R = typename Raw<TIn>::type;
    extern __shared__ float smem[];
    float *sA = smem, *sB = smem + S * CW, *sP = smem + 2 * S * CW, *sI = smem + 3 * S * CW;

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
        sA[idx] = sum[q].a;
        sB[idx] = sum[q].b;
        sP[idx] = sum[q].p;
    }
    __syncthreads();

    // Phase C: one lane per channel scans the S summaries (exclusive, from the tile start),
    // then fetches the tile's incoming state.
    if (tid < CW) {
        const int ch = tid;
        const int64_t c = ct * CW + ch;
        const bool cok = c < a.C;
        const float wc = cok ? a.w[c] : 0.f;
        St run = st_empty();
        for (int jj = 0; jj < S; ++jj) {
            const int64_t len = std::max<int64_t>(0, std::min<int64_t>(L, a.T - (tile_t0 + (int64_t)jj * L)));
            const int idx = jj * CW + ch;
            const St cur = St{sA[idx], sB[idx], sP[idx]};
            sA[idx] = run.a;
            sB[idx] = run.b;
            sP[idx] = run.p;
            run = combine(run, cur, span_decay(len, wc));
        }
        St prefix = st_empty();
        if (tt == 0 && a.state_in && cok) {
            const int64_t s = b * a.C + c;
            prefix = St{a.state_in[s], a.state_in[BC + s], a.state_in[2 * BC + s]};
        }
        if (nTT > 1 && tt < nTT - 1) {
            const int64_t chain = (b * nCT + ct) * nTT;
            if (tt > 0) {
                publish(ws, chain + tt, kAgg, run, ch);
                prefix = lookback(ws, chain, tt, wc, TW, ch);
            }
            publish(ws, chain + tt, kIncl, combine(prefix, run, span_decay(tile_len, wc)), ch);
        } else if (nTT > 1) {
            prefix = lookback(ws, (b * nCT + ct) * nTT, tt, wc, TW, ch);
        }
        sI[ch] = prefix.a;
        sI[CW + ch] = prefix.b;
        sI[2 * CW + ch] = prefix.p;
    }
    __syncthreads();

    // Phase D: the lane's starting state = tile prefix, then the sub-chunks before it.
    St st[4];
    const int64_t before = std::min<int64_t>((int64_t)j * L, tile_len);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cl = g * 4 + q;
        const St pre = St{sI[cl], sI[CW + cl], sI[2 * CW + cl]};
        const St exl = St{sA[j * CW + cl], sB[j * CW + cl], sP[j * CW + cl]};
        st[q] = combine(pre, exl, span_decay(before, w[q]));
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
                emit(st[q], u[q], kk, vv, num, den);
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
                    a.state_out[2 * BC + sc + q] = st[q].p;
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
    const size_t lds = (size_t)(3 * S * kTileChannels + 3 * kTileChannels) * sizeof(float);
    if (blocks > 0x7fffffff || 16 * S > chunk_max_threads<TIn, MODE>()) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((wkv_chunk_kernel<TIn, TOut, MODE>), dim3((unsigned)blocks), dim3(16 * S), lds,
                       s, a, ws, S, nCT, nTT, chunk_len);
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
    // flags [tiles][64] u32 + agg, incl [tiles][3][64] f32 + one error word, 256-B aligned parts
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    return (size_t)(al(tiles * kTileChannels * 4) + 2 * al(tiles * 3 * kTileChannels * 4) + 256);
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
    p += al(tiles * 3 * kTileChannels * 4);
    ws->incl = reinterpret_cast<float *>(p);
    p += al(tiles * 3 * kTileChannels * 4);
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
