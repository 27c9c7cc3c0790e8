// stream_ceiling.hip -- bandwidth ceilings for the benchmark (libwkvceiling.so, not part of
// librwkvwkv): kernels that move exactly the bytes of a WKV launch, in the same launch shape and
// with the same memory instructions, but do no arithmetic and wait for nothing.  The time one
// takes is what the memory system allows that access pattern; the WKV kernel's time above it is
// the cost of its arithmetic and of its dependencies.
//
//   wkvceil_tile    the chunked scan's pattern: one workgroup of 4 waves per (batch row, 64-channel
//                   tile, time tile of 4 x L tokens), blockIdx time-tile-major, the (batch row,
//                   channel tile) of an index chosen as the scan chooses it (with 8 XCDs and a
//                   multiple of 8 channel tiles, each XCD takes a contiguous range, rotated from
//                   one time tile to the next when the grid exceeds one resident round); each wave copies
//                   its L rows of every input into LDS with 16-byte global-to-LDS loads carrying
//                   the non-temporal hint, waits, and writes its L rows of the output from LDS
//                   with 16-byte non-temporal stores.  The LDS size is the scan kernel's, so the
//                   same number of workgroups share a CU.
//   wkvceil_lanes   the sequential (decode) kernel's pattern: one lane per (batch row, 4
//                   channels); non-temporal vector loads of the activations (4 channels each)
//                   and of the three state planes (16 bytes each), the same stores back.
//   wkvceil_stream  a grid-stride stream of plain 16-byte loads and stores over the same bytes
//                   (no LDS, no hints): the simplest pattern, for context.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));

constexpr int kTileChannels = 64;

__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 2);
}

// esz_in / esz_out: element bytes (2 or 4); n_in inputs (up to 3), one output.
__global__ void __launch_bounds__(256) tile_kernel(const char *in0, const char *in1, const char *in2, int n_in,
                                                   char *out, int64_t B, int64_t T, int64_t C, int L, int esz_in,
                                                   int esz_out, int lds_rows, int rot) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nCT = (int)((C + kTileChannels - 1) / kTileChannels);
    const int64_t BCT = B * nCT;
    const int TW = 4 * L;
    const int64_t tt = blockIdx.x / BCT, rem = blockIdx.x - tt * BCT;
    // workgroup i runs on XCD i mod 8: index rem takes chain (rem % 8) * (BCT / 8) + rem / 8 when
    // nCT is a multiple of 8, so that each XCD reads a contiguous range of channel tiles
    const int64_t r = (nCT % 8 == 0) ? ((rem + (rot ? tt : 0)) % 8) * (BCT / 8) + rem / 8 : rem;
    const int64_t b = r / nCT, ct = r - b * nCT;
    const int64_t t0 = tt * TW + (int64_t)wv * L;
    const char *src[3] = {in0, in1, in2};
    // inputs: rows of 64 * esz_in bytes in chunks of 16; rows per instruction = 64 / chunks
    const int chunks_in = kTileChannels * esz_in / 16, rpi_in = 64 / chunks_in;
    const int q = lane % chunks_in, rs = lane / chunks_in;
    const int64_t row_in = C * esz_in;
    for (int j = 0; j < L; j += rpi_in)
        for (int s = 0; s < n_in; ++s) {
            const int64_t t = min(t0 + j + rs, T - 1);
            const char *g = src[s] + (b * T + t) * row_in + ct * kTileChannels * esz_in + q * 16;
            char *l = smem + ((size_t)s * lds_rows + wv * L + j) * kTileChannels * esz_in;
            dma16(g, l);
        }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // output rows from the first input's staged rows (same bytes when the sizes agree, else the
    // first half of them twice: the data is not the point)
    const int chunks_out = kTileChannels * esz_out / 16, rpi_out = 64 / chunks_out;
    const int qo = lane % chunks_out, ro = lane / chunks_out;
    const int64_t row_out = C * esz_out;
    const int stage_bytes = kTileChannels * esz_in;
    for (int j = 0; j < L; j += rpi_out) {
        const int64_t t = t0 + j + ro;
        if (t < T) {
            const f4 v = *reinterpret_cast<const f4 *>(smem + ((size_t)(wv * L + j + ro)) * stage_bytes +
                                                        (qo * 16) % stage_bytes);
            __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(out + (b * T + t) * row_out +
                                                                  ct * kTileChannels * esz_out + qo * 16));
        }
    }
}

// One lane per 4 channels of a batch row: n_act activation inputs of esz bytes (8 bytes per lane
// at esz 2), one activation output, and (with state) three fp32 planes read and written.
__global__ void __launch_bounds__(256) lanes_kernel(const char *a0, const char *a1, const char *a2, int n_act,
                                                    char *y, float *state, int64_t n4, int esz) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const char *src[3] = {a0, a1, a2};
    i2 acc = {0, 0};
    f4 acc4 = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_act; ++s) {
        if (esz == 2) {
            const i2 v = __builtin_nontemporal_load(reinterpret_cast<const i2 *>(src[s]) + i);
            acc = acc ^ v;
        } else {
            const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(src[s]) + i);
            acc4 = acc4 + v;
        }
    }
    if (state) {
        f4 *st = reinterpret_cast<f4 *>(state);
        const f4 s0 = __builtin_nontemporal_load(st + i), s1 = __builtin_nontemporal_load(st + n4 + i),
                 s2 = __builtin_nontemporal_load(st + 2 * n4 + i);
        __builtin_nontemporal_store(s1, st + i);
        __builtin_nontemporal_store(s2, st + n4 + i);
        __builtin_nontemporal_store(s0, st + 2 * n4 + i);
    }
    if (esz == 2)
        __builtin_nontemporal_store(acc, reinterpret_cast<i2 *>(y) + i);
    else
        __builtin_nontemporal_store(acc4, reinterpret_cast<f4 *>(y) + i);
}

// Grid-stride: every 16-byte chunk of the output is the xor of the inputs' chunks at the same
// index (inputs and output of equal size in 16-byte units, n16 of them).
__global__ void __launch_bounds__(256) stream_kernel(const f4 *a0, const f4 *a1, const f4 *a2, int n_in, f4 *y,
                                                     int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
        f4 acc = a0[i];
        if (n_in > 1) acc = acc + a1[i];
        if (n_in > 2) acc = acc + a2[i];
        y[i] = acc;
    }
}

}  // namespace

extern "C" {

// The chunked scan's pattern over [B, T, C]: n_in inputs of esz_in bytes, one output of esz_out
// bytes, tiles of 64 channels x 4 waves x L tokens, lds_bytes of LDS per workgroup (the scan
// kernel's, for its occupancy).  C must be a multiple of 64 / esz (whole 16-byte chunks).
int wkvceil_tile(const void *in0, const void *in1, const void *in2, int n_in, void *out, int64_t B, int64_t T,
                 int64_t C, int L, int esz_in, int esz_out, int lds_bytes, hipStream_t s) {
    if (n_in < 1 || n_in > 3 || (C % 64) != 0 || (L != 16 && L != 32) || (esz_in != 2 && esz_in != 4) ||
        (esz_out != 2 && esz_out != 4) || lds_bytes < n_in * 4 * L * 64 * esz_in)
        return -1;
    const int64_t grid = B * (C / 64) * ((T + 4 * L - 1) / (4 * L));
    int per_cu = 0, cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tile_kernel, 256, lds_bytes) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -4;
    const int rot = grid > (int64_t)per_cu * cus ? 1 : 0;  // more than one resident round
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)grid), dim3(256), lds_bytes, s, (const char *)in0,
                       (const char *)in1, (const char *)in2, n_in, (char *)out, B, T, C, L, esz_in, esz_out, 4 * L,
                       rot);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// The sequential kernel's pattern over n elements (n % 4 == 0): n_act activation inputs and one
// output of esz bytes per element, and the [3][n] fp32 state read and written when state is set.
int wkvceil_lanes(const void *a0, const void *a1, const void *a2, int n_act, void *y, float *state, int64_t n,
                  int esz, hipStream_t s) {
    if (n_act < 1 || n_act > 3 || (n % 4) != 0 || (esz != 2 && esz != 4)) return -1;
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(lanes_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, (const char *)a0,
                       (const char *)a1, (const char *)a2, n_act, (char *)y, state, n4, esz);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// A plain grid-stride stream: n_in inputs and one output of bytes each (a multiple of 16).
int wkvceil_stream(const void *a0, const void *a1, const void *a2, int n_in, void *y, int64_t bytes, int blocks,
                   hipStream_t s) {
    if (n_in < 1 || n_in > 3 || (bytes % 16) != 0 || blocks < 1) return -1;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const f4 *)a0, (const f4 *)a1,
                       (const f4 *)a2, n_in, (f4 *)y, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
