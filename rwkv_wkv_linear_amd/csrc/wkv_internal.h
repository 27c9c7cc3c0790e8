// wkv_internal.h -- internal interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace rwkvwkv {

// Workgroup barrier for an exchange through LDS alone: each wave waits for its own LDS
// accesses (lgkmcnt) and nothing else.  __syncthreads() also makes every global load and store
// of the wave complete first (vmcnt(0)), which would stall on loads still streaming in;
// global-to-LDS loads are not covered here, so a reader of another wave's staged rows needs
// that wave to have waited for them (vmcnt) before the barrier.  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt(63) and expcnt(7) do not wait
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

enum Mode : int {
    MODE_PLAIN = 0,    // y = wkv
    MODE_GATED = 1,    // y = sigmoid(r) * wkv, r a [B,T,C] tensor
    MODE_TIMEMIX = 2,  // token shift prologue, r = xr, y = sigmoid(xr) * wkv
};

// Everything a forward launch needs; pointers are device memory.
struct ForwardArgs {
    int64_t B, T, C;
    const float *w, *u;
    const void *k, *v;
    const void *r;                       // MODE_GATED
    const void *x, *x_prev;              // MODE_TIMEMIX (x_prev may be null)
    const float *mix_k, *mix_v, *mix_r;  // MODE_TIMEMIX
    void *xk_out, *xv_out, *x_last;      // MODE_TIMEMIX, each may be null
    void *y;
    const float *state_in;  // may be null (empty state)
    float *state_out;       // may be null
    int in_dt, out_dt;  // rwkv_dtype codes: 0 fp32, 1 fp16, 2 bf16
    int mode;
    int publish;  // rwkv_publish: how look-back states are published (single-pass chunked scan)
    int vec;    // 1: C % 4 == 0 and activation pointers aligned for 4-element vectors
    int vec16;   // 1: input rows split into 16-byte chunks (C % (16 / size) == 0, 16-B aligned)
    int vec16y;  // 1: the same for y
    int vecs;    // 1: C % 4 == 0 and both state pointers 16-byte aligned (float4 state I/O)
    int vecp;    // 1: C % 4 == 0 and every per-channel parameter pointer 16-byte aligned
};

// Chunked-scan scratch: per tile and channel four 64-bit words (a, b, key, age), each the
// fp32 value tagged with (epoch << 2 | kind) in its high half.
struct ChunkWorkspace {
    uint64_t *words;  // single pass: [tiles][4][64] tagged words
    float *aggs;      // two passes: [tiles][64][4] tile aggregates
    uint32_t *err;    // one word, nonzero once a look-back wait gave up (that launch's epoch),
                      // until rwkv4_lookback_status clears it
    uint32_t epoch;   // per-launch stamp; words of other launches never match
};

constexpr int kTileChannels = 64;  // channels per workgroup tile
constexpr int kMinChunk = 16, kMaxChunk = 1024;

// Longest tile staged in LDS at once (160 KB of rows and wave summaries): for 2-byte inputs 512
// tokens ungated and 256 gated or time mix (a third tensor of rows), for fp32 half of those.
// The two-pass scan takes chunk lengths up to it; the single-launch scan runs longer chunks
// (up to kMaxChunk) as long tiles of 4-wave sub-tiles.
int tile_max_len(int in_2byte, int gated);
// Chunk length (tokens per workgroup tile) the auto policy picks for a shape.
int auto_chunk_len(int64_t B, int64_t T, int64_t C, int in_2byte);
// True when the auto policy picks the sequential kernel.
bool auto_sequential(int64_t B, int64_t T, int64_t C);
// Workspace layout for a chunked launch.
size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t C, int chunk_len);
void chunk_workspace_carve(void *base, int64_t B, int64_t T, int64_t C, int chunk_len,
                           ChunkWorkspace *ws);

// Per input dtype (the kernels of each are compiled in their own translation unit).
hipError_t launch_sequential_in0(const ForwardArgs &a, hipStream_t s);
hipError_t launch_sequential_in1(const ForwardArgs &a, hipStream_t s);
hipError_t launch_sequential_in2(const ForwardArgs &a, hipStream_t s);
hipError_t launch_chunked_in0(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s);
hipError_t launch_chunked_in1(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s);
hipError_t launch_chunked_in2(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s);
hipError_t launch_chunked_2pass_in0(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s);
hipError_t launch_chunked_2pass_in1(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s);
hipError_t launch_chunked_2pass_in2(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws, hipStream_t s);

hipError_t launch_sequential(const ForwardArgs &a, hipStream_t s);
hipError_t launch_chunked(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws,
                          hipStream_t s);
// Two launches: tile aggregates, then every tile folds its predecessors' aggregates.
hipError_t launch_chunked_2pass(const ForwardArgs &a, int chunk_len, const ChunkWorkspace &ws,
                                hipStream_t s);
// Longest chain (time tiles per (b, channel tile)) the two-pass scan takes by default: none.
// Measured on the 14B layer shape, the two launches take 19.8 us against 12.7 us for the
// single pass with its look-back, so AUTO keeps the single pass; RWKV_ALGO_TWO_PASS stays
// available (graph-capturable, no cross-workgroup waiting).
constexpr int kTwoPassMaxTiles = 0;
// T == 0: state_out <- state_in (or the empty state), x_last <- x_prev (or zeros).
hipError_t launch_passthrough(const ForwardArgs &a, hipStream_t s);

// Pre-LN token-shift prologue (mix_kernels.hip).
struct ShiftMixArgs {
    int64_t B, T, C;
    const void *x, *x_prev;
    void *x_last;
    const float *ln_weight, *ln_bias;  // ln_weight null: no LayerNorm
    float ln_eps;
    const float *mix[3];  // k, v, r; each may be null
    void *out[3];         // xk, xv, xr; null exactly when its mix is
    int dt;               // rwkv_dtype code of x, x_prev, x_last and the outputs
    int vec;              // 1: C % 8 == 0 and every pointer 16-byte aligned
};
hipError_t launch_shift_mix(const ShiftMixArgs &a, hipStream_t s);

// Channel-mix receptance gate (mix_kernels.hip): y = residual + kv / (1 + e^{-r}).
struct GateLaunch {
    int64_t n;
    const void *r, *kv, *residual;  // residual may be null
    void *y;
    int in_dt, out_dt;
    int vec;  // 1: n % 8 == 0 and every pointer 16-byte aligned
};
hipError_t launch_gate(const GateLaunch &g, hipStream_t s);

}  // namespace rwkvwkv
