// Internal declarations shared by the host library and the kernel translation
// units.  Not part of the public C ABI (that is include/deltalog.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dl {

// Slot ids travel to the device inside the kernel argument block, so a launch
// carries at most this many decoded slots; larger calls are split on the host.
constexpr int kMaxLaunchSlots = 512;

// Largest log capacity C = L - 1 (sizes the per-block coefficient arrays).
constexpr int kMaxLogCap = 63;

// A launch's slot word: the slot id in the low 24 bits; a decode launch puts
// the host's live length of the slot (<= kMaxLogCap) in the top 8, so that one
// scalar argument load brings both.
constexpr int kSlotBits = 24;
constexpr uint32_t kSlotMask = (1u << kSlotBits) - 1;
constexpr int kMaxSlots = 1 << kSlotBits;
// Top byte of a decode launch's slot word when the host gives no live length
// (launches recorded into a graph, whose replays may start at any phase).
constexpr uint32_t kNoHint = 0xFF;
// StepParams::slot0 of a launch whose blocks read their slot words.
constexpr uint32_t kGathered = 0xFFFFFFFFu;

enum Mode : int {
    MODE_STEP = 0,   // DeltaLog decode: append, or merge when the log is full
    MODE_EAGER = 1,  // eager read-modify-write of the dense state (no log)
    MODE_MERGE = 2,  // materialize base + log, no token
    MODE_STEP_SPLIT = 3,  // MODE_STEP whose appending units read ReplayPrep's coefficients
    MODE_REPLAY_PREP = 4, // ReplayPrep: key-side coefficients once per (entry, v-head)
    MODE_STEP_CONSEC = 5, // MODE_STEP over consecutive slots (slot0, slot0 + 1, ..), no host live lengths
};

enum DType : int { F32 = 0, BF16 = 1 };
enum Decay : int { DECAY_NONE = 0, DECAY_SCALAR = 1, DECAY_PER_KEY = 2 };

// Arguments of the decode / eager / merge kernels.  Token-side pointers are
// already offset to this launch's first batch entry.
struct StepParams {
    void *base;          // [P, H_v, NV, D, BV]  state dtype, value-tile major
    void *klog;          // [P, H_k, C, D]       input dtype
    void *ulog;          // [P, H_v, C, D]       fp32 (delta) | input dtype (plain)
    float *lamlog;       // [P, H_v, C] | [P, H_v, C, D]
    int32_t *nlog;       // [P, H_v, NV] live length per value tile
    const void *q;       // [n, H_k, D]
    const void *k;       // [n, H_k, D]
    const void *v;       // [n, H_v, D]
    const float *lam;    // [n, H_v] | [n, H_v, D]
    const float *beta;   // [n, H_v]
    float *out;          // [n, H_v, D]
    float *coef;         // [n, H_v, 2 (C + 1)] replay coefficients (split replay only)
    int32_t H_v;
    int32_t H_k;
    int32_t C;           // log capacity L - 1
    int32_t NV;          // value tiles per slot-head
    int32_t nunits;      // blocks in this launch = n * H_v * (d_v / B_V), or n * H_v (ReplayPrep)
    uint32_t slot0;      // first slot of a MODE_STEP_CONSEC launch, else kGathered
    uint32_t slots[kMaxLaunchSlots];   // slot words (see kSlotBits)
};

// Largest number of steps one window call carries.
constexpr int kMaxWindow = 4096;

// Arguments of the window kernel: W consecutive decode steps of the same
// slots, the state of each block's tile held in registers from the first step
// to the last.  Token arrays are step-major, [W][B][..]; the pointers are
// offset to this launch's first batch entry and B is the call's batch (the
// stride between steps).
struct WindowParams {
    void *base;          // [P, H_v, NV, D, BV]  state dtype, value-tile major
    const void *klog;    // [P, H_k, C, D]       input dtype
    const void *ulog;    // [P, H_v, C, D]       fp32 (delta) | input dtype (plain)
    const float *lamlog; // [P, H_v, C] | [P, H_v, C, D]
    int32_t *nlog;       // [P, H_v, NV]
    const void *q;       // [W, B, H_k, D]
    const void *k;       // [W, B, H_k, D]
    const void *v;       // [W, B, H_v, D]
    const float *lam;    // [W, B, H_v] | [W, B, H_v, D]
    const float *beta;   // [W, B, H_v]
    float *out;          // [W, B, H_v, D]
    int32_t H_v;
    int32_t H_k;
    int32_t C;           // log capacity L - 1
    int32_t NV;          // value tiles per slot-head
    int32_t nunits;      // blocks in this launch = n * H_v * NV
    int32_t W;           // steps
    int32_t B;           // entries per step in the token arrays
    uint32_t slots[kMaxLaunchSlots];   // slot ids
};

// Arguments of the state-copy kernel (slot assignment and base read-back):
// whole-slot state copies between the caller's natural layout [n, H_v, D, D]
// and the pool's value-tile-major base [P, H_v, NV, D, BV].
struct CopyParams {
    void *base;          // [P, H_v, NV, D, BV]
    int32_t *nlog;       // [P, H_v, NV]
    void *ext;           // [n, H_v, D, D] natural layout; NULL = zero state (to the pool only)
    int32_t to_pool;     // 1: ext -> base and empty the log (assign); 0: base -> ext (read)
    int32_t row_vecs;    // 16-byte vectors per natural row (D * sizeof(state) / 16)
    int32_t tile_vecs;   // 16-byte vectors per tile row (BV * sizeof(state) / 16)
    int32_t D;
    int32_t H_v;
    int32_t NV;          // value tiles per slot-head (live-length counters per slot-head)
    int32_t nunits;      // n * H_v
    int32_t slots[kMaxLaunchSlots];
};

// Dynamic LDS of a decode / merge block: the live log as stored, back to
// back -- key factors [n][D] (input type), value factors on the block's tile
// [n][BV] (fp32 for delta updates, else input type) and, for per-key decay,
// the snapshots [n][D] (fp32) -- sized for a full log.  Pools whose log would
// need more than kMaxLogStageBytes are refused.
constexpr size_t kMaxLogStageBytes = 56 * 1024;
inline size_t log_stage_bytes(int D, int BV, int C, int decay, int update, int in_dtype) {
    const size_t s_in = in_dtype == BF16 ? 2 : 4;
    const size_t s_b = update != 0 ? 4 : s_in;
    return (size_t)C * (D * s_in + BV * s_b + (decay == DECAY_PER_KEY ? D * sizeof(float) : 0));
}

// Default value-tile width, by the number of slot-heads a launch may carry
// (max_batch * H_v).  Once they fill the GPU with blocks, whole-row tiles: one
// block per slot-head streams its state and replays its log once.  For fp32
// d = 128 this measured up to 3.5% faster per step than 64-column tiles with
// per-key decay and up to 3% with scalar decay at B <= 64, and level beyond,
// although the wider tile holds 3 waves per SIMD instead of 5.  Smaller
// launches spread one step over more CUs with narrower tiles: 16 columns for
// 63 slot-heads or fewer at d = 128 (about 2% faster than 32 for 32
// slot-heads), then 32, and for fp32 d = 128 also 64 below 256 slot-heads, so
// that a launch keeps at least 256 blocks.  A bf16 state with a log (L > 1)
// and a scalar or no decay takes 64 columns up to 2047 slot-heads: half-size
// tiles double the blocks of a launch that is one round of whole rows, which
// measured 8% faster per step at 1024 slot-heads and 1.6% at 2048 (GDN,
// d = 128), while fp32 states and the eager kernel (L = 1) measured the same
// or faster with whole rows.
inline int default_value_tile(int D, int state_dtype, long long units, int decay, int L) {
    if (D < 64) return D;
    if (D == 128 && units < 64) return 16;
    if (D == 128 && state_dtype != BF16 && units >= 128 && units < 256) return 64;
    if (units < 256) return 32;
    if (D == 128 && state_dtype == BF16 && L > 1 && decay != DECAY_PER_KEY && units < 2048) return 64;
    return D;
}
// The window kernel stages token inputs in LDS kWindowChunk steps at a time,
// double buffered: per buffer q, a [K][D], e^{lambda} [K][D] (per-key decay),
// v [K][BV], then e^{lambda} (scalar), beta and a . q per step.
constexpr int kWindowChunk = 8;
inline size_t window_token_floats(int D, int BV, int decay) {
    return (size_t)kWindowChunk * (2 * D + (decay == DECAY_PER_KEY ? D : 0) + BV + 4);
}
inline size_t window_stage_bytes(int D, int BV, int C, int decay, int update, int in_dtype) {
    const size_t tok = 2 * window_token_floats(D, BV, decay) * sizeof(float);
    const size_t log = log_stage_bytes(D, BV, C, decay, update, in_dtype);
    return tok > log ? tok : log;
}

inline bool value_tile_supported(int D, int BV) {
    switch (D) {
    case 128: return BV == 128 || BV == 64 || BV == 32 || BV == 16;
    case 64: return BV == 64 || BV == 32;
    case 32: return BV == 32;
    case 16: return BV == 16;
    default: return false;
    }
}

// Launch one decode / eager / merge kernel; returns hipError_t as int.
int launch_step(int D, int BV, int mode, int decay, int update, int state_dtype, int in_dtype,
                const StepParams &p, size_t shmem, hipStream_t stream);

int launch_copy(const CopyParams &p, hipStream_t stream);

// Launch one window kernel; returns hipError_t as int.
int launch_window(int D, int BV, int decay, int update, int state_dtype, int in_dtype, const WindowParams &p,
                  size_t shmem, hipStream_t stream);

}  // namespace dl
