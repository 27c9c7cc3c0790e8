// mix_kernels.hip -- gfx950 kernels for the mixers' elementwise prologue and epilogue.
//
// Pre-LN token-shift prologue (rwkv4_shift_mix).  The "RWKV-4 14B" page, Facts table, places a
// LayerNorm before each mixer (ln1 before time mixing, ln2 before channel mixing); the port
// report's Abstract lists pre-LN and the token shift that mixes the current and the previous
// token.  Per batch row b and token t:
//
//   n_t    = LayerNorm(x_t) = (x_t - mean_t) / sqrt(var_t + eps) * weight + bias   (or x_t)
//   out_t  = mix * n_t + (1 - mix) * n_{t-1},   n_{-1} = x_prev (already normalised)
//
// for up to three mixes (time mixing: k, v, r; channel mixing: k, r), and x_last = n_{T-1}.
// mean_t and the biased variance var_t run over the C channels of the row.
//
// Channel-mix receptance gate (rwkv4_channelmix_gate): y = residual + kv / (1 + e^{-r})
// (the port report's "channel-mix gating"; the 14B page's field table gives channel mixing its
// own receptance matrix).
//
// Both are streaming kernels bound by HBM: the prologue reads x once from HBM (the row
// statistics pass) and re-reads it from L2, and writes each requested output once.

#include "wkv_internal.h"

#include <algorithm>

namespace rwkvwkv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowsPerBlock = 4;  // output rows per prologue workgroup (plus the row before them)
// Rows of at most 1024 chunks of 8 take the single-read kernel (shift_mix_row_kernel, one
// thread per chunk).  Wider rows take shift_mix_kernel with the threads below: one per chunk up
// to 1024 for 2-byte data and 512 for fp32 (whose chunks hold twice the registers), the rest
// looping, and at least a wave per statistics row.
template <typename T> constexpr int shift_max_threads() { return sizeof(T) == 4 ? 512 : 1024; }
template <typename T> int shift_threads(int64_t C) {
    const int64_t want = ((C + 7) / 8 + 63) / 64 * 64;
    return (int)std::min<int64_t>(shift_max_threads<T>(), std::max<int64_t>(64 * (kRowsPerBlock + 1), want));
}
static_assert(64 * (kRowsPerBlock + 1) <= 512, "a wave per statistics row");

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { using type = h8; };
template <> struct Vec8<__bf16> { using type = b8; };

// 8 consecutive elements starting at p: one 16-byte load (two for fp32) when vec, else
// per-element loads of the first cnt (the rest read as 0).
// With NT the loads carry the non-temporal (streaming) hint: for data read for the last time.
template <typename V, bool NT>
__device__ __forceinline__ V ldv(const V *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <typename T, bool NT = false>
__device__ __forceinline__ void ld8(const T *p, bool vec, int cnt, float (&f)[8]) {
    if (vec) {
        if constexpr (sizeof(T) == 4) {
            const f4v a = ldv<f4v, NT>(reinterpret_cast<const f4v *>(p)), b = ldv<f4v, NT>(reinterpret_cast<const f4v *>(p) + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[i] = a[i];
                f[4 + i] = b[i];
            }
        } else {
            const typename Vec8<T>::type a = ldv<typename Vec8<T>::type, NT>(reinterpret_cast<const typename Vec8<T>::type *>(p));
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = (float)a[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = i < cnt ? (float)ldv<T, NT>(p + i) : 0.f;
    }
}

// Outputs are written once and never read back by the launch: streaming (non-temporal) stores,
// so the lines do not linger dirty in L2 for the end-of-kernel write-back.
template <typename V>
__device__ __forceinline__ void st_stream(V *p, V v) {
    __builtin_nontemporal_store(v, p);
}

// Store of 8 elements, rounded to nearest-even for 2-byte types.
template <typename T>
__device__ __forceinline__ void st8(T *p, bool vec, int cnt, const float (&f)[8]) {
    if (vec) {
        if constexpr (sizeof(T) == 4) {
            f4v a, b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = f[i];
                b[i] = f[4 + i];
            }
            st_stream(reinterpret_cast<f4v *>(p), a);
            st_stream(reinterpret_cast<f4v *>(p) + 1, b);
        } else {
            typename Vec8<T>::type a;
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = (T)f[i];
            st_stream(reinterpret_cast<typename Vec8<T>::type *>(p), a);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < cnt) st_stream(p + i, (T)f[i]);
    }
}

// 8 consecutive elements kept in their storage type (4 VGPRs for 2-byte types), converted to
// fp32 on use; loads as ld8.
template <typename T> struct Raw8 {
    typename Vec8<T>::type v;
    __device__ __forceinline__ float operator[](int i) const { return (float)v[i]; }
};
template <> struct Raw8<float> {
    f4v a, b;
    __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

template <typename T, bool NT = false>
__device__ __forceinline__ Raw8<T> ldraw(const T *p, bool vec, int cnt) {
    Raw8<T> r;
    if constexpr (sizeof(T) == 4) {
        if (vec) {
            r.a = ldv<f4v, NT>(reinterpret_cast<const f4v *>(p));
            r.b = ldv<f4v, NT>(reinterpret_cast<const f4v *>(p) + 1);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                r.a[i] = i < cnt ? ldv<float, NT>(p + i) : 0.f;
                r.b[i] = 4 + i < cnt ? ldv<float, NT>(p + 4 + i) : 0.f;
            }
        }
    } else {
        if (vec) {
            r.v = ldv<typename Vec8<T>::type, NT>(reinterpret_cast<const typename Vec8<T>::type *>(p));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) r.v[i] = i < cnt ? ldv<T, NT>(p + i) : T(0);
        }
    }
    return r;
}

// Running (count, mean, sum of squared deviations) of a set of values; two sets merge
// exactly in real arithmetic by Chan, Golub and LeVeque's pairwise update, which keeps the
// deviations small (no E[x^2] - E[x]^2 cancellation).
struct Moments {
    float n, mean, m2;
};

__device__ __forceinline__ Moments merge(const Moments &a, const Moments &b) {
    if (b.n == 0.f) return a;
    if (a.n == 0.f) return b;
    const float n = a.n + b.n;
    const float d = b.mean - a.mean;
    const float fb = b.n / n;
    return Moments{n, fmaf(d, fb, a.mean), a.m2 + b.m2 + d * d * a.n * fb};
}

// Sum over the 64 lanes of a wave by cross-lane moves within each row of 16 lanes (DPP: swap
// neighbours, swap pairs, mirror the half rows, mirror the row), after which every lane of a row
// holds the row's sum; the four row sums are then read as scalars and added in a fixed order, so
// every lane returns the same value.  No LDS round trips, unlike the butterfly of shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_rows(float v) {
    v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);  // row_half_mirror
    v += dpp_move<0x140>(v);  // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Moments of one row of C values, reduced over the 64 lanes of the calling wave; every lane
// returns the row's result.
template <typename T>
__device__ Moments row_moments(const T *row, int64_t C, bool vec, int lane) {
    // chunks in flight per lane: 8192 (2-byte) or 4096 (fp32) channels per pass
    constexpr int NF = sizeof(T) == 2 ? 16 : 8;
    const int64_t nchunks = (C + 7) / 8;
    // The row streams through in passes of NF chunks per lane (every chunk's own mean and
    // squared deviations, exact over its 8 values), merged pairwise.
    Moments acc{0.f, 0.f, 0.f};
    for (int64_t j0 = 0; j0 < nchunks; j0 += NF * 64) {
        Raw8<T> f[NF];
        int cnt[NF];
#pragma unroll
        for (int m = 0; m < NF; ++m) {
            const int64_t j = j0 + m * 64 + lane;
            cnt[m] = j < nchunks ? (int)std::min<int64_t>(8, C - 8 * j) : 0;
            if (cnt[m] > 0) f[m] = ldraw(row + 8 * j, vec, cnt[m]);
        }
#pragma unroll
        for (int m = 0; m < NF; ++m) {
            if (cnt[m] > 0) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) s += f[m][i];  // padding reads as 0
                const float cn = (float)cnt[m];
                const float mu = s / cn;
                float q = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float d = f[m][i] - mu;
                    if (i < cnt[m]) q = fmaf(d, d, q);
                }
                acc = merge(acc, Moments{cn, mu, q});
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const Moments o{__shfl_xor(acc.n, off), __shfl_xor(acc.mean, off), __shfl_xor(acc.m2, off)};
        // the lower lane of each pair keeps its own moments first, so both lanes form the same
        // merge and stay identical
        acc = (lane & off) ? merge(o, acc) : merge(acc, o);
    }
    return acc;
}

struct ShiftArgs {
    int64_t B, T, C;
    const void *x, *x_prev;
    void *x_last;
    const float *ln_w, *ln_b;
    float eps;
    const float *mix[3];  // k, v, r (each may be null)
    void *out[3];         // xk, xv, xr (null exactly when the mix is)
    int vec;              // C % 8 == 0 and every pointer 16-byte aligned
};

// Rows wider than 1024 chunks: workgroup (b, rows t0 .. t0+3), shift_threads<T>(C) threads.  Phase 1 (LayerNorm only): wave
// w <= 4 takes the statistics of row t0 - 1 + w (wave 0 of the first block takes row T - 1 instead, for x_last)
// and puts (mean, 1/sqrt(var + eps)) in LDS.  Phase 2: each thread takes 8-channel chunks; per
// chunk it issues every load first (parameters, the previous row or x_prev, its rows, and the
// last row for x_last), then normalises the rows in order, keeping the previous normalised row
// in registers, and writes the mixes.  The first block of each batch row also writes x_last,
// after it has read x_prev, so x_last may be x_prev itself.
template <typename T, bool LN>
__global__ void __launch_bounds__(shift_max_threads<T>()) shift_mix_kernel(ShiftArgs a) {
    __shared__ float s_mean[kRowsPerBlock + 1], s_rstd[kRowsPerBlock + 1];
    const int64_t nTB = std::max<int64_t>(1, (a.T + kRowsPerBlock - 1) / kRowsPerBlock);
    const int64_t b = blockIdx.x / nTB;
    const int64_t t0 = (blockIdx.x - b * nTB) * kRowsPerBlock;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t C = a.C;
    const bool vec = a.vec != 0;
    const T *X = static_cast<const T *>(a.x);
    const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(kRowsPerBlock, a.T - t0));
    const bool want_last = t0 == 0 && a.x_last != nullptr;

    if constexpr (LN) {
        int64_t s = -1;
        if (wv == 0)
            s = t0 > 0 ? t0 - 1 : (want_last && a.T > 0 ? a.T - 1 : -1);
        else if (wv <= rows)
            s = t0 + wv - 1;
        if (s >= 0) {
            const Moments m = row_moments(X + (b * a.T + s) * C, C, vec, lane);
            if (lane == 0) {
                s_mean[wv] = m.mean;
                s_rstd[wv] = 1.f / sqrtf(m.m2 / (float)C + a.eps);
            }
        }
        __syncthreads();
    }

    const int64_t nchunks = (C + 7) / 8;
    for (int64_t j = threadIdx.x; j < nchunks; j += blockDim.x) {
        const int64_t c0 = 8 * j;
        const int cnt = (int)std::min<int64_t>(8, C - c0);
        // every load of the chunk first: one memory latency per chunk
        float g[8], be[8], mx[3][8];
        if constexpr (LN) {
            ld8(a.ln_w + c0, vec, cnt, g);
            if (a.ln_b)
                ld8(a.ln_b + c0, vec, cnt, be);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) be[i] = 0.f;
        }
#pragma unroll
        for (int m = 0; m < 3; ++m)
            if (a.mix[m]) ld8(a.mix[m] + c0, vec, cnt, mx[m]);
        const T *col = X + b * a.T * C + c0;
        Raw8<T> xr[kRowsPerBlock], xp, xl;
#pragma unroll
        for (int r = 0; r < kRowsPerBlock; ++r)
            if (r < rows) xr[r] = ldraw<T, true>(col + (t0 + r) * C, vec, cnt);  // the rows' last reads
        if (t0 > 0)
            xp = ldraw(col + (t0 - 1) * C, vec, cnt);
        else if (a.x_prev)
            xp = ldraw(static_cast<const T *>(a.x_prev) + b * C + c0, vec, cnt);
        if (want_last && a.T > 0) xl = ldraw(col + (a.T - 1) * C, vec, cnt);

        // normalised chunk of a row (statistics in LDS slot k)
        auto norm = [&](const Raw8<T> &raw, int k, float (&o)[8]) {
            if constexpr (LN) {
                const float mu = s_mean[k], rs = s_rstd[k];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = fmaf((raw[i] - mu) * rs, g[i], be[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = raw[i];
            }
        };
        float prev[8];
        if (t0 > 0) {
            norm(xp, 0, prev);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) prev[i] = a.x_prev ? xp[i] : 0.f;
        }
        if (want_last) {
            // x_last: the normalised last row, or x_prev when there are no tokens
            float last[8];
            if (a.T > 0) {
                norm(xl, 0, last);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) last[i] = prev[i];
            }
            st8(static_cast<T *>(a.x_last) + b * C + c0, vec, cnt, last);
        }
#pragma unroll
        for (int r = 0; r < kRowsPerBlock; ++r) {
            if (r < rows) {
                float cur[8];
                norm(xr[r], r + 1, cur);
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    if (a.mix[m]) {
                        float o[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) o[i] = fmaf(mx[m][i], cur[i] - prev[i], prev[i]);
                        st8(static_cast<T *>(a.out[m]) + (b * a.T + t0 + r) * C + c0, vec, cnt, o);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) prev[i] = cur[i];
            }
        }
    }
}

// Single-read form for rows of at most 1024 chunks of 8 (every thread holds one chunk of each
// row): workgroup (b, rows t0 .. t0+3) with one thread per chunk.  Each thread loads its chunk
// of five rows once (slot 0: the row before t0, or row T - 1 in the first block, which writes
// x_last; slots 1..4: the block's rows), then the statistics run as a pipeline over the slots.
// Stage k reduces the squared deviations of slot k - 1 (about its mean, from stage k - 1) and
// the sum of slot k through one LDS exchange and one barrier, and then writes the outputs of
// slot k - 1, so a row's outputs leave while the later rows are still landing.  The reductions
// are the two-pass textbook ones: per-thread chunk sums, a butterfly of plain adds per wave,
// then the wave partials added in wave order (every thread forms the same sums).
template <typename T, bool LN>
__global__ void __launch_bounds__(1024) shift_mix_row_kernel(ShiftArgs a) {
    constexpr int R = kRowsPerBlock;
    __shared__ float s_sum[R + 1][16], s_sq[R + 1][16];
    const int64_t nTB = std::max<int64_t>(1, (a.T + R - 1) / R);
    const int64_t b = blockIdx.x / nTB;
    const int64_t t0 = (blockIdx.x - b * nTB) * R;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nW = blockDim.x >> 6;
    const int64_t C = a.C;
    const bool vec = a.vec != 0;
    const T *X = static_cast<const T *>(a.x);
    const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(R, a.T - t0));
    const bool want_last = t0 == 0 && a.x_last != nullptr;
    // slot 0: the row before t0, else (first block) the last row for x_last; block-uniform
    const int64_t s0row = t0 > 0 ? t0 - 1 : (want_last && a.T > 0 ? a.T - 1 : -1);
    auto slot_valid = [&](int k) { return k == 0 ? s0row >= 0 : k - 1 < rows; };

    const int64_t nchunks = (C + 7) / 8;
    const int64_t j = threadIdx.x;
    const int64_t c0 = 8 * j;
    const int cnt = j < nchunks ? (int)std::min<int64_t>(8, C - c0) : 0;
    const T *col = X + b * a.T * C + c0;
    // loads in the order they are needed: slot 0, x_prev, the parameters, then the rows
    Raw8<T> xs[R + 1], xp;
    float g[8], be[8], mx[3][8];
    if (cnt > 0) {
        if (s0row >= 0) xs[0] = ldraw(col + s0row * C, vec, cnt);
        if (t0 == 0 && a.x_prev) xp = ldraw(static_cast<const T *>(a.x_prev) + b * C + c0, vec, cnt);
        if constexpr (LN) {
            ld8(a.ln_w + c0, vec, cnt, g);
            if (a.ln_b)
                ld8(a.ln_b + c0, vec, cnt, be);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) be[i] = 0.f;
        }
#pragma unroll
        for (int m = 0; m < 3; ++m)
            if (a.mix[m]) ld8(a.mix[m] + c0, vec, cnt, mx[m]);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < rows) xs[r + 1] = ldraw<T, true>(col + (t0 + r) * C, vec, cnt);  // last reads
    }

    const float ic = 1.f / (float)C;
    float mean[R + 1], rstd[R + 1], prev[8];
#pragma unroll
    for (int k = 0; k <= R + 1; ++k) {
        if constexpr (LN) {
            // stage k: squared deviations of slot k - 1 and the sum of slot k
            const bool dq = k >= 1 && slot_valid(k - 1), dm = k <= R && slot_valid(k);
            if (dq) {
                float q = 0.f;
                if (cnt > 0) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float d = xs[k - 1][i] - mean[k - 1];
                        if (i < cnt) q = fmaf(d, d, q);
                    }
                }
                q = wave_sum_rows(q);
                if (lane == 0) s_sq[k - 1][wv] = q;
            }
            if (dm) {
                float p = 0.f;  // padding reads as 0
                if (cnt > 0) {
                    const Raw8<T> &f = xs[k];
                    p = ((f[0] * ic + f[1] * ic) + (f[2] * ic + f[3] * ic)) + ((f[4] * ic + f[5] * ic) + (f[6] * ic + f[7] * ic));
                }
                p = wave_sum_rows(p);
                if (lane == 0) s_sum[k][wv] = p;
            }
            if (dq || dm) lds_barrier();  // the outputs of earlier slots stay in flight
            if (dq) {
                float v = 0.f;
                for (int w = 0; w < nW; ++w) v += s_sq[k - 1][w];
                rstd[k - 1] = 1.f / sqrtf(v / (float)C + a.eps);
            }
            if (dm) {
                float m = 0.f;
                for (int w = 0; w < nW; ++w) m += s_sum[k][w];
                mean[k] = m;
            }
        }
        if (k == 0 || cnt == 0) continue;
        // outputs of slot k - 1
        const int sl = k - 1;
        auto norm = [&](const Raw8<T> &raw, float (&o)[8]) {
            if constexpr (LN) {
                const float mu = mean[sl], rs = rstd[sl];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = fmaf((raw[i] - mu) * rs, g[i], be[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = raw[i];
            }
        };
        if (sl == 0) {
            if (t0 > 0) {
                norm(xs[0], prev);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) prev[i] = a.x_prev ? xp[i] : 0.f;
                if (want_last) {
                    // x_last: the normalised last row, or x_prev when there are no tokens (x_prev
                    // was read above, so x_last may be x_prev itself)
                    float last[8];
                    if (a.T > 0) {
                        norm(xs[0], last);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) last[i] = prev[i];
                    }
                    st8(static_cast<T *>(a.x_last) + b * C + c0, vec, cnt, last);
                }
            }
        } else if (sl - 1 < rows) {
            float cur[8];
            norm(xs[sl], cur);
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                if (a.mix[m]) {
                    float o[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[i] = fmaf(mx[m][i], cur[i] - prev[i], prev[i]);
                    st8(static_cast<T *>(a.out[m]) + (b * a.T + t0 + sl - 1) * C + c0, vec, cnt, o);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) prev[i] = cur[i];
        }
    }
}

struct GateArgs {
    int64_t n;
    const void *r, *kv, *res;
    void *y;
    int vec;  // n % 8 == 0 and every pointer 16-byte aligned
};

// y = residual + kv / (1 + e^{-r}); grid-stride over 8-element chunks.
template <typename TIn, typename TOut>
__global__ void __launch_bounds__(256) gate_kernel(GateArgs a) {
    const TIn *R = static_cast<const TIn *>(a.r);
    const TIn *KV = static_cast<const TIn *>(a.kv);
    const TIn *RES = static_cast<const TIn *>(a.res);
    TOut *Y = static_cast<TOut *>(a.y);
    const bool vec = a.vec != 0;
    const int64_t nchunks = (a.n + 7) / 8;
    for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < nchunks;
         j += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i0 = 8 * j;
        const int cnt = (int)std::min<int64_t>(8, a.n - i0);
        float r[8], kv[8], res[8], y[8];
        ld8<TIn, true>(R + i0, vec, cnt, r);
        ld8<TIn, true>(KV + i0, vec, cnt, kv);
        if (RES) ld8<TIn, true>(RES + i0, vec, cnt, res);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float g = kv[i] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * r[i]));
            y[i] = RES ? res[i] + g : g;
        }
        st8(Y + i0, vec, cnt, y);
    }
}

template <typename T>
hipError_t launch_shift_t(const ShiftArgs &a, hipStream_t s) {
    const int64_t nTB = std::max<int64_t>(1, (a.T + kRowsPerBlock - 1) / kRowsPerBlock);
    const dim3 grid((unsigned)(a.B * nTB));
    const int64_t nchunks = (a.C + 7) / 8;
    if (nchunks <= 1024) {
        // one thread per chunk, whole waves
        const dim3 block((unsigned)std::max<int64_t>(64, (nchunks + 63) / 64 * 64));
        if (a.ln_w)
            hipLaunchKernelGGL((shift_mix_row_kernel<T, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((shift_mix_row_kernel<T, false>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (a.ln_w)
        hipLaunchKernelGGL((shift_mix_kernel<T, true>), grid, dim3(shift_threads<T>(a.C)), 0, s, a);
    else
        hipLaunchKernelGGL((shift_mix_kernel<T, false>), grid, dim3(shift_threads<T>(a.C)), 0, s, a);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_gate_t(const GateArgs &a, int out_dt, unsigned blocks, hipStream_t s) {
    if (out_dt == 1) hipLaunchKernelGGL((gate_kernel<TIn, _Float16>), dim3(blocks), dim3(256), 0, s, a);
    else if (out_dt == 2) hipLaunchKernelGGL((gate_kernel<TIn, __bf16>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gate_kernel<TIn, float>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shift_mix(const ShiftMixArgs &m, hipStream_t s) {
    ShiftArgs a{};
    a.B = m.B;
    a.T = m.T;
    a.C = m.C;
    a.x = m.x;
    a.x_prev = m.x_prev;
    a.x_last = m.x_last;
    a.ln_w = m.ln_weight;
    a.ln_b = m.ln_bias;
    a.eps = m.ln_eps;
    for (int i = 0; i < 3; ++i) {
        a.mix[i] = m.mix[i];
        a.out[i] = m.out[i];
    }
    a.vec = m.vec;
    if (m.dt == 1) return launch_shift_t<_Float16>(a, s);
    if (m.dt == 2) return launch_shift_t<__bf16>(a, s);
    return launch_shift_t<float>(a, s);
}

hipError_t launch_gate(const GateLaunch &g, hipStream_t s) {
    GateArgs a{g.n, g.r, g.kv, g.residual, g.y, g.vec};
    const int64_t nchunks = (g.n + 7) / 8;
    // enough workgroups to fill the chip several times over; the loop covers the rest
    const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((nchunks + 255) / 256, 8192));
    if (g.in_dt == 1) return launch_gate_t<_Float16>(a, g.out_dt, blocks, s);
    if (g.in_dt == 2) return launch_gate_t<__bf16>(a, g.out_dt, blocks, s);
    return launch_gate_t<float>(a, g.out_dt, blocks, s);
}

}  // namespace rwkvwkv
