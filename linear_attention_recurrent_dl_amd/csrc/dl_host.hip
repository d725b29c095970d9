// Host side of the DeltaLog C ABI (include/deltalog.h): pool descriptor
// validation, buffer sizing, the host mirror of every slot's live-log length
// (the append / merge schedule of [DL]'s append-merge cycle), slot
// assignment, and kernel launches.
//
// [DL] = "DeltaLog: Deferred Materialization of Recurrent States for Linear
// Attention Decoding".  The phase of a decoded slot follows its design
// section: a slot whose log holds C = L - 1 entries takes the merge step,
// any other appends at index n.  The serving-integration section's allocator
// gives a fresh slot the supplied base and an empty log.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "deltalog.h"
#include "dl_internal.hpp"
#include "dl_mirror.hpp"

namespace dl {
template <int D, int BV>
hipError_t launch_step_d(int, int, int, int, int, const StepParams &, size_t, hipStream_t);
template <int D, int BV>
hipError_t launch_window_d(int, int, int, int, const WindowParams &, size_t, hipStream_t);
}

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DL_OK;
}

size_t dtype_size(int dt) { return dt == DL_BF16 ? 2 : 4; }

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int value_tile_of(const dl_pool_desc *d) {
    if (d->value_tile) return d->value_tile;
    int bv = dl::default_value_tile(d->d_k, d->state_dtype, (long long)d->max_batch * d->num_v_heads, d->decay,
                                    d->merge_interval);
    // a default whose live log would not fit the LDS staging budget falls back
    // to the widest narrower tile that does (the value factors shrink with it)
    while (dl::value_tile_supported(d->d_k, bv / 2) &&
           dl::log_stage_bytes(d->d_k, bv, d->merge_interval - 1, d->decay, d->update, d->in_dtype) >
               dl::kMaxLogStageBytes)
        bv /= 2;
    return bv;
}

int validate_desc(const dl_pool_desc *d) {
    if (!d) return fail(DL_ERR_INVALID_ARG, "desc is NULL");
    if (d->num_slots < 1 || d->num_slots > dl::kMaxSlots)
        return fail(DL_ERR_INVALID_ARG, "num_slots must be in [1, %d] (got %d)", dl::kMaxSlots, d->num_slots);
    if (d->max_batch < 1) return fail(DL_ERR_INVALID_ARG, "max_batch must be >= 1 (got %d)", d->max_batch);
    if (d->num_v_heads < 1 || d->num_k_heads < 1)
        return fail(DL_ERR_INVALID_ARG, "head counts must be >= 1 (H_v=%d, H_k=%d)", d->num_v_heads, d->num_k_heads);
    if (d->num_v_heads % d->num_k_heads)
        return fail(DL_ERR_INVALID_ARG, "num_v_heads (%d) must be a multiple of num_k_heads (%d)",
                    d->num_v_heads, d->num_k_heads);
    // the kernels take a v-head's q/k head as the high word of
    // 2h * ceil(2^31 / (H_v / H_k)), exact while h * (H_v / H_k) < 2^31
    if (d->num_v_heads > 32768)
        return fail(DL_ERR_INVALID_ARG, "num_v_heads (%d) must be at most 32768", d->num_v_heads);
    if (d->merge_interval < 1 || d->merge_interval > dl::kMaxLogCap + 1)
        return fail(DL_ERR_INVALID_ARG, "merge_interval must be in [1, %d] (got %d)", dl::kMaxLogCap + 1,
                    d->merge_interval);
    if (d->decay < DL_DECAY_NONE || d->decay > DL_DECAY_PER_KEY) return fail(DL_ERR_INVALID_ARG, "bad decay %d", d->decay);
    if (d->update < DL_UPDATE_PLAIN || d->update > DL_UPDATE_DELTA) return fail(DL_ERR_INVALID_ARG, "bad update %d", d->update);
    if ((d->state_dtype != DL_F32 && d->state_dtype != DL_BF16) || (d->in_dtype != DL_F32 && d->in_dtype != DL_BF16))
        return fail(DL_ERR_INVALID_ARG, "bad dtype (state %d, in %d)", d->state_dtype, d->in_dtype);
    if (d->d_k != d->d_v || !supported_dim(d->d_k))
        return fail(DL_ERR_UNSUPPORTED, "head dims d_k=%d d_v=%d not built (need d_k == d_v in {16,32,64,128})",
                    d->d_k, d->d_v);
    if (d->replay_split != 0 && d->replay_split != 1)
        return fail(DL_ERR_INVALID_ARG, "replay_split must be 0 or 1 (got %d)", d->replay_split);
    if (d->value_tile != 0 && !dl::value_tile_supported(d->d_k, d->value_tile))
        return fail(DL_ERR_UNSUPPORTED, "value_tile %d not built for d=%d", d->value_tile, d->d_k);
    const int bv = value_tile_of(d);
    if (dl::log_stage_bytes(d->d_k, bv, d->merge_interval - 1, d->decay, d->update, d->in_dtype) > dl::kMaxLogStageBytes)
        return fail(DL_ERR_UNSUPPORTED, "merge_interval %d with d=%d needs %zu B of LDS for the live log (limit %zu)",
                    d->merge_interval, d->d_k,
                    dl::log_stage_bytes(d->d_k, bv, d->merge_interval - 1, d->decay, d->update, d->in_dtype),
                    dl::kMaxLogStageBytes);
    const long long units = (long long)d->max_batch * d->num_v_heads;
    if (units > (1LL << 30)) return fail(DL_ERR_INVALID_ARG, "max_batch * num_v_heads too large");
    // the kernels index (slot, v-head, value tile) in 32 bits
    if ((long long)d->num_slots * d->num_v_heads * (d->d_k / bv) > (1LL << 31) - 1)
        return fail(DL_ERR_INVALID_ARG, "num_slots * num_v_heads * (d / value_tile) must be below 2^31");
    return DL_OK;
}

void compute_sizes(const dl_pool_desc *d, size_t out[DL_NUM_BUFS]) {
    const size_t P = d->num_slots, Hv = d->num_v_heads, Hk = d->num_k_heads, D = d->d_k;
    const size_t C = d->merge_interval - 1;
    const size_t b_size = d->update == DL_UPDATE_DELTA ? 4 : dtype_size(d->in_dtype);
    const size_t lam_w = d->decay == DL_DECAY_PER_KEY ? D : 1;
    out[DL_BUF_BASE] = P * Hv * D * D * dtype_size(d->state_dtype);
    out[DL_BUF_KLOG] = P * Hk * C * D * dtype_size(d->in_dtype);
    out[DL_BUF_ULOG] = P * Hv * C * D * b_size;
    out[DL_BUF_LAMLOG] = d->decay == DL_DECAY_NONE ? 0 : P * Hv * C * lam_w * 4;
    out[DL_BUF_NLOG] = P * Hv * (D / value_tile_of(d)) * 4;
    // replay coefficients of one launch: 2 (C + 1) floats per (entry, v-head)
    const size_t launch_slots = std::min<size_t>(d->max_batch, dl::kMaxLaunchSlots);
    out[DL_BUF_COEF] = (d->replay_split && C > 0) ? launch_slots * Hv * 2 * (C + 1) * 4 : 0;
}

__global__ void dl_zero_i32_kernel(int32_t *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

// Whole-slot state copies, one block per (slot, v-head), in 16-byte vectors.
// Vector i of a slot-head in the pool's tile-major base is (tile vt, row r,
// vector cv of the tile row); in the natural layout it sits at row r, vector
// vt * tile_vecs + cv.  Assignment (to_pool) also empties the slot's log.
__global__ void __launch_bounds__(256) dl_copy_state_kernel(const dl::CopyParams p) {
    const int unit = blockIdx.x;
    const int j = unit / p.H_v, h = unit - j * p.H_v;
    const size_t sh = (size_t)p.slots[j] * p.H_v + h;
    const int tv = p.tile_vecs, tile_v = p.D * tv;
    const int nvec = p.D * p.row_vecs;
    uint4 *pool = reinterpret_cast<uint4 *>(p.base) + sh * nvec;
    uint4 *ext = p.ext ? reinterpret_cast<uint4 *>(p.ext) + (size_t)unit * nvec : nullptr;
    for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
        const int vt = i / tile_v, rem = i - vt * tile_v;
        const int r = rem / tv, cv = rem - r * tv;
        const int nat = r * p.row_vecs + vt * tv + cv;
        if (p.to_pool) pool[i] = ext ? ext[nat] : make_uint4(0, 0, 0, 0);
        else ext[nat] = pool[i];
    }
    if (p.to_pool && threadIdx.x < (unsigned)p.NV) p.nlog[sh * p.NV + threadIdx.x] = 0;
}

}  // namespace

namespace dl {

int launch_step(int D, int BV, int mode, int decay, int update, int st, int it, const StepParams &p, size_t shmem,
                hipStream_t s) {
#define DL_TILE(d_, bv_) \
    if (D == d_ && BV == bv_) return (int)launch_step_d<d_, bv_>(mode, decay, update, st, it, p, shmem, s);
    DL_TILE(128, 128) DL_TILE(128, 64) DL_TILE(128, 32) DL_TILE(128, 16)
    DL_TILE(64, 64) DL_TILE(64, 32) DL_TILE(32, 32) DL_TILE(16, 16)
#undef DL_TILE
    return (int)hipErrorInvalidValue;
}

int launch_window(int D, int BV, int decay, int update, int st, int it, const WindowParams &p, size_t shmem,
                  hipStream_t s) {
#define DL_TILE(d_, bv_) \
    if (D == d_ && BV == bv_) return (int)launch_window_d<d_, bv_>(decay, update, st, it, p, shmem, s);
    DL_TILE(128, 128) DL_TILE(128, 64) DL_TILE(128, 32) DL_TILE(128, 16)
    DL_TILE(64, 64) DL_TILE(64, 32) DL_TILE(32, 32) DL_TILE(16, 16)
#undef DL_TILE
    return (int)hipErrorInvalidValue;
}

int launch_copy(const CopyParams &p, hipStream_t s) {
    dl_copy_state_kernel<<<dim3(p.nunits), dim3(256), 0, s>>>(p);
    return (int)hipGetLastError();
}

}  // namespace dl

struct dl_pool {
    dl_pool_desc desc;
    dl_pool_buffers buf;
    int bv;                         // value-tile width B_V
    int nv;                         // value tiles per slot-head
    bool dry;                       // host-only pool: validate + mirror, no device work
    std::vector<int32_t> n;         // host mirror of live-log length per slot
    bool stale;                     // a call was recorded into a graph: replays move the
                                    // device counters without the mirror
    std::vector<uint32_t> seen;     // duplicate detection (generation stamps)
    uint32_t gen;
};

namespace {

int check_slots(dl_pool *pool, int32_t B, const int32_t *ids) {
    if (B < 0) return fail(DL_ERR_INVALID_ARG, "negative count %d", B);
    if (B > pool->desc.max_batch)
        return fail(DL_ERR_BATCH_TOO_LARGE, "batch %d exceeds max_batch %d", B, pool->desc.max_batch);
    if (B > 0 && !ids) return fail(DL_ERR_INVALID_ARG, "slot_ids is NULL");
    if (++pool->gen == 0) {           // stamp wrapped: clear and restart
        std::fill(pool->seen.begin(), pool->seen.end(), 0u);
        pool->gen = 1;
    }
    for (int32_t j = 0; j < B; ++j) {
        const int32_t s = ids[j];
        if (s < 0 || s >= pool->desc.num_slots)
            return fail(DL_ERR_SLOT_RANGE, "slot id %d at position %d outside [0, %d)", s, j, pool->desc.num_slots);
        if (pool->seen[s] == pool->gen) return fail(DL_ERR_DUPLICATE_SLOT, "slot id %d repeated (position %d)", s, j);
        pool->seen[s] = pool->gen;
    }
    return DL_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(DL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Whether work enqueued on `stream` now is recorded into a graph instead of
// run.  A call recorded into a graph marks the pool's mirror stale: its
// replays move the device counters and the mirror does not follow them.
bool capturing(dl_pool *pool, void *stream) {
    if (pool->dry) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    bool cap = true;                            // unknown: assume recorded
    if (hipStreamIsCapturing((hipStream_t)stream, &cs) == hipSuccess)
        cap = cs != hipStreamCaptureStatusNone;
    else
        (void)hipGetLastError();
    if (cap) pool->stale = true;
    return cap;
}

// Natural-layout states in or out of the pool's tile-major base, split into
// launches of at most kMaxLaunchSlots slots.  ext: [n, H_v, d_k, d_v].
int copy_states(dl_pool *pool, int32_t n, const int32_t *ids, void *ext, bool to_pool, void *stream) {
    const dl_pool_desc &d = pool->desc;
    const size_t esz = dtype_size(d.state_dtype);
    const size_t head_bytes = (size_t)d.d_k * d.d_v * esz;
    dl::CopyParams p;
    memset(&p, 0, sizeof p);
    p.base = pool->buf.base;
    p.nlog = pool->buf.nlog;
    p.to_pool = to_pool ? 1 : 0;
    p.row_vecs = (int32_t)(d.d_v * esz / 16);
    p.tile_vecs = (int32_t)(pool->bv * esz / 16);
    p.D = d.d_k;
    p.H_v = d.num_v_heads;
    p.NV = pool->nv;
    auto launch = [&](int32_t lo, int32_t cnt) -> int {
        if (pool->dry) return hipSuccess;
        p.ext = ext ? static_cast<char *>(ext) + (size_t)lo * d.num_v_heads * head_bytes : nullptr;
        p.nunits = cnt * d.num_v_heads;
        memcpy(p.slots, ids + lo, cnt * sizeof(int32_t));
        return dl::launch_copy(p, (hipStream_t)stream);
    };
    auto commit = [&](int32_t lo, int32_t cnt) {
        if (to_pool) dl::mirror_clear(pool->n.data(), ids + lo, cnt);
    };
    return dl::launch_chunks(n, dl::kMaxLaunchSlots, launch, commit);
}

// First slot of a launch whose cnt slots are consecutive, else kGathered
// (its blocks then read their slot words).
uint32_t consecutive_slot0(const int32_t *ids, int32_t cnt) {
    for (int32_t j = 1; j < cnt; ++j)
        if (ids[j] != ids[0] + j) return dl::kGathered;
    return (uint32_t)ids[0];
}

// Shared by dl_decode_step, dl_eager_step and dl_decode_step_noalloc.  The
// split-replay coefficients of a launch go to `coef` (the pool's buffer, or
// the static scratch), launches carry at most `chunk` slots.
int decode(dl_pool *pool, int32_t B, const int32_t *ids, const void *q, const void *a_or_k, const void *b_or_v,
           const float *lambda, const float *beta, float *out, void *stream, bool eager_call,
           float *coef = nullptr, int32_t chunk = dl::kMaxLaunchSlots) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    const dl_pool_desc &d = pool->desc;
    if (eager_call && d.merge_interval != 1)
        return fail(DL_ERR_INVALID_ARG, "dl_eager_step needs a pool with merge_interval == 1 (got %d)", d.merge_interval);
    int rc = check_slots(pool, B, ids);
    if (rc) return rc;
    if (d.decay == DL_DECAY_NONE && lambda) return fail(DL_ERR_INVALID_ARG, "lambda must be NULL for DL_DECAY_NONE");
    if (d.update == DL_UPDATE_PLAIN && beta) return fail(DL_ERR_INVALID_ARG, "beta must be NULL for DL_UPDATE_PLAIN");
    if (B == 0) return ok();
    if (!pool->dry) {
        if (!q || !a_or_k || !b_or_v || !out) return fail(DL_ERR_INVALID_ARG, "NULL q / a_or_k / b_or_v / out");
        if (d.decay != DL_DECAY_NONE && !lambda) return fail(DL_ERR_INVALID_ARG, "lambda is NULL");
        if (d.update == DL_UPDATE_DELTA && !beta) return fail(DL_ERR_INVALID_ARG, "beta is NULL");
        const uintptr_t align = (uintptr_t)q | (uintptr_t)a_or_k | (uintptr_t)b_or_v | (uintptr_t)out;
        if (align & 15) return fail(DL_ERR_INVALID_ARG, "token buffers must be 16-byte aligned");

        const int C = d.merge_interval - 1;
        const bool split = d.replay_split && C > 0;
        const int mode = C == 0 ? dl::MODE_EAGER : (split ? dl::MODE_STEP_SPLIT : dl::MODE_STEP);
        const size_t D = d.d_k, Hv = d.num_v_heads, Hk = d.num_k_heads, s_in = dtype_size(d.in_dtype);
        const size_t lam_w = d.decay == DL_DECAY_PER_KEY ? D : 1;
        const size_t shmem = dl::log_stage_bytes(d.d_k, pool->bv, C, d.decay, d.update, d.in_dtype);
        if (!coef) coef = pool->buf.coef;
        if (split && !coef)
            return fail(DL_ERR_INVALID_ARG, "split-replay pool created without a coefficient buffer: "
                                            "decode it with dl_decode_step_noalloc");
        // A launch recorded into a graph may be replayed at any phase of the
        // append-merge cycle, so it carries no live lengths from the host.
        const bool cap = capturing(pool, stream);
        dl::StepParams p;
        memset(&p, 0, sizeof p);
        p.base = pool->buf.base;
        p.klog = pool->buf.klog;
        p.ulog = pool->buf.ulog;
        p.lamlog = pool->buf.lamlog;
        p.nlog = pool->buf.nlog;
        p.coef = coef;
        p.H_v = d.num_v_heads;
        p.H_k = d.num_k_heads;
        p.C = C;
        p.NV = pool->nv;
        auto launch = [&](int32_t lo, int32_t cnt) -> int {
            p.q = static_cast<const char *>(q) + (size_t)lo * Hk * D * s_in;
            p.k = static_cast<const char *>(a_or_k) + (size_t)lo * Hk * D * s_in;
            p.v = static_cast<const char *>(b_or_v) + (size_t)lo * Hv * D * s_in;
            p.lam = lambda ? lambda + (size_t)lo * Hv * lam_w : nullptr;
            p.beta = beta ? beta + (size_t)lo * Hv : nullptr;
            p.out = out + (size_t)lo * Hv * D;
            memcpy(p.slots, ids + lo, cnt * sizeof(int32_t));
            if (mode == dl::MODE_STEP) {         // the host's live lengths ride in the slot words
                for (int32_t j = 0; j < cnt; ++j)
                    p.slots[j] |= (cap ? dl::kNoHint : (uint32_t)pool->n[ids[lo + j]]) << dl::kSlotBits;
            }
            // A recorded decode launch of consecutive slots names its first:
            // the blocks then know their slots without an argument fetch.  A
            // direct one keeps its slot words, which carry the host's live
            // lengths.
            p.slot0 = (mode == dl::MODE_STEP && cap) ? consecutive_slot0(ids + lo, cnt) : dl::kGathered;
            const int kmode = p.slot0 != dl::kGathered ? dl::MODE_STEP_CONSEC : mode;
            if (split) {
                // ReplayPrep, one block per (entry, v-head), into the coefficient scratch
                p.nunits = cnt * d.num_v_heads;
                const int e = dl::launch_step(d.d_k, pool->bv, dl::MODE_REPLAY_PREP, d.decay, d.update,
                                              d.state_dtype, d.in_dtype, p, shmem, (hipStream_t)stream);
                if (e != hipSuccess) return hip_fail((hipError_t)e, "replay-prep kernel launch");
            }
            p.nunits = cnt * d.num_v_heads * pool->nv;
            const int e = dl::launch_step(d.d_k, pool->bv, kmode, d.decay, d.update, d.state_dtype, d.in_dtype, p,
                                          shmem, (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail((hipError_t)e, "decode kernel launch");
            return DL_OK;
        };
        auto commit = [&](int32_t lo, int32_t cnt) { dl::mirror_decode(pool->n.data(), ids + lo, cnt, C); };
        rc = dl::launch_chunks(B, chunk, launch, commit);
        return rc ? rc : ok();
    }
    dl::mirror_decode(pool->n.data(), ids, B, d.merge_interval - 1);
    return ok();
}

// Standalone merges of the given (validated, distinct) slots.  Every slot is
// launched: a block whose device counter reads 0 exits at once, so the set
// does not depend on the host mirror, which a graph replay leaves behind.
int merge_slots(dl_pool *pool, int32_t n, const int32_t *ids, void *stream) {
    const dl_pool_desc &d = pool->desc;
    const int C = d.merge_interval - 1;
    if (!pool->dry) (void)capturing(pool, stream);
    dl::StepParams p;
    memset(&p, 0, sizeof p);
    p.base = pool->buf.base;
    p.klog = pool->buf.klog;
    p.ulog = pool->buf.ulog;
    p.lamlog = pool->buf.lamlog;
    p.nlog = pool->buf.nlog;
    p.H_v = d.num_v_heads;
    p.H_k = d.num_k_heads;
    p.C = C;
    p.NV = pool->nv;
    const size_t shmem = dl::log_stage_bytes(d.d_k, pool->bv, C, d.decay, d.update, d.in_dtype);
    auto launch = [&](int32_t lo, int32_t cnt) -> int {
        if (pool->dry || C == 0) return DL_OK;     // no log to merge in an eager pool
        p.nunits = cnt * d.num_v_heads * pool->nv;
        memcpy(p.slots, ids + lo, cnt * sizeof(int32_t));
        p.slot0 = dl::kGathered;
        const int e = dl::launch_step(d.d_k, pool->bv, dl::MODE_MERGE, d.decay, d.update, d.state_dtype,
                                      d.in_dtype, p, shmem, (hipStream_t)stream);
        return e != hipSuccess ? hip_fail((hipError_t)e, "merge kernel launch") : DL_OK;
    };
    auto commit = [&](int32_t lo, int32_t cnt) { dl::mirror_clear(pool->n.data(), ids + lo, cnt); };
    const int rc = dl::launch_chunks(n, dl::kMaxLaunchSlots, launch, commit);
    return rc ? rc : ok();
}

}  // namespace

extern "C" {

int dl_pool_sizes(const dl_pool_desc *desc, size_t bytes_out[DL_NUM_BUFS]) {
    int rc = validate_desc(desc);
    if (rc) return rc;
    if (!bytes_out) return fail(DL_ERR_INVALID_ARG, "bytes_out is NULL");
    compute_sizes(desc, bytes_out);
    return ok();
}

int dl_pool_create(const dl_pool_desc *desc, const dl_pool_buffers *buffers, dl_pool **out) {
    int rc = validate_desc(desc);
    if (rc) return rc;
    if (!out) return fail(DL_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    size_t sz[DL_NUM_BUFS];
    compute_sizes(desc, sz);
    if (buffers) {
        const void *ptrs[DL_NUM_BUFS] = {buffers->base, buffers->klog, buffers->ulog, buffers->lamlog, buffers->nlog,
                                         buffers->coef};
        for (int i = 0; i < DL_NUM_BUFS; ++i) {
            // the coefficient scratch may be left out: such a pool decodes
            // through dl_decode_step_noalloc, whose scratch is the library's
            if (sz[i] && !ptrs[i] && i != DL_BUF_COEF)
                return fail(DL_ERR_INVALID_ARG, "buffer %d is NULL but needs %zu bytes", i, sz[i]);
            if ((uintptr_t)ptrs[i] & 15) return fail(DL_ERR_INVALID_ARG, "buffer %d is not 16-byte aligned", i);
        }
    }
    dl_pool *p = new (std::nothrow) dl_pool;
    if (!p) return fail(DL_ERR_INVALID_ARG, "out of host memory");
    p->desc = *desc;
    p->bv = value_tile_of(desc);
    p->nv = desc->d_k / p->bv;
    p->dry = buffers == nullptr;
    if (buffers) p->buf = *buffers;
    else memset(&p->buf, 0, sizeof p->buf);
    p->n.assign(desc->num_slots, 0);
    p->seen.assign(desc->num_slots, 0u);
    p->gen = 0;
    p->stale = false;
    if (!p->dry) {
        const size_t cnt = sz[DL_BUF_NLOG] / 4;
        const int blocks = (int)std::min<size_t>((cnt + 255) / 256, 4096);
        dl_zero_i32_kernel<<<dim3(blocks), dim3(256), 0, 0>>>(p->buf.nlog, cnt);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess) e = hipStreamSynchronize(0);
        if (e != hipSuccess) {
            delete p;
            return hip_fail(e, "clearing log lengths");
        }
    }
    *out = p;
    return ok();
}

int dl_pool_destroy(dl_pool *pool) {
    delete pool;
    return ok();
}

int dl_slot_assign(dl_pool *pool, int32_t n, const int32_t *slot_ids, const void *init_base, void *stream) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_slots(pool, n, slot_ids);
    if (rc) return rc;
    if (init_base && ((uintptr_t)init_base & 15)) return fail(DL_ERR_INVALID_ARG, "init_base is not 16-byte aligned");
    if (n == 0) return ok();
    (void)capturing(pool, stream);
    // the mirror is cleared launch by launch (a host-only pool launches nothing)
    const int e = copy_states(pool, n, slot_ids, const_cast<void *>(init_base), true, stream);
    if (e != hipSuccess) return hip_fail((hipError_t)e, "assign kernel launch");
    return ok();
}

int dl_read_base(dl_pool *pool, int32_t n, const int32_t *slot_ids, void *out, void *stream) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_slots(pool, n, slot_ids);
    if (rc) return rc;
    if (pool->dry) return fail(DL_ERR_DRY_RUN, "host-only pool has no device state");
    if (n == 0) return ok();
    if (!out) return fail(DL_ERR_INVALID_ARG, "out is NULL");
    if ((uintptr_t)out & 15) return fail(DL_ERR_INVALID_ARG, "out is not 16-byte aligned");
    const int e = copy_states(pool, n, slot_ids, out, false, stream);
    if (e != hipSuccess) return hip_fail((hipError_t)e, "read kernel launch");
    return ok();
}

int dl_decode_step(dl_pool *pool, int32_t B, const int32_t *slot_ids, const void *q, const void *a_or_k,
                   const void *b_or_v, const float *lambda, const float *beta, float *out, void *stream) {
    return decode(pool, B, slot_ids, q, a_or_k, b_or_v, lambda, beta, out, stream, false);
}

int dl_eager_step(dl_pool *pool, int32_t B, const int32_t *slot_ids, const void *q, const void *a_or_k,
                  const void *b_or_v, const float *lambda, const float *beta, float *out, void *stream) {
    return decode(pool, B, slot_ids, q, a_or_k, b_or_v, lambda, beta, out, stream, true);
}

// ---- the entry point that allocates nothing -------------------------------
//
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops) decode split-replay pools through dl_decode_step_noalloc: the
// replay coefficients go to this file-scope array instead of the pool's
// coefficient buffer.  Each GPU holds its own copy from the library's load
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not a device address: its device address is looked up once per device and
// only that pointer is handed to kernels.
}  // extern "C"

namespace {

constexpr size_t kScratchFloats = size_t(1) << 20;          // 4 MiB per device
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices];

// Device address of the current device's `scratch`, looked up on the first
// call made with that device current.
int scratch_address(float **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DL_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev,
                                                  kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return DL_OK;
}

}  // namespace

extern "C" {

int dl_decode_step_noalloc(dl_pool *pool, int32_t B, const int32_t *slot_ids, const void *q, const void *a_or_k,
                           const void *b_or_v, const float *lambda, const float *beta, float *out, void *stream) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    const dl_pool_desc &d = pool->desc;
    const int C = d.merge_interval - 1;
    if (!(d.replay_split && C > 0))            // no kernel of this pool uses a scratch buffer
        return decode(pool, B, slot_ids, q, a_or_k, b_or_v, lambda, beta, out, stream, false);
    // one slot's coefficients: 2 (C + 1) floats per v-head; a launch carries
    // as many slots as the scratch holds (at most the usual launch limit)
    const size_t per_slot = (size_t)d.num_v_heads * 2 * (C + 1);
    if (per_slot > kScratchFloats)
        return fail(DL_ERR_UNSUPPORTED, "one slot's replay coefficients need %zu floats, more than the %zu of the "
                                        "static scratch (num_v_heads * 2 * merge_interval <= %zu)",
                    per_slot, kScratchFloats, kScratchFloats);
    const int32_t chunk = (int32_t)std::min<size_t>(dl::kMaxLaunchSlots, kScratchFloats / per_slot);
    float *ptr = nullptr;
    if (!pool->dry) {
        const int rc = scratch_address(&ptr);
        if (rc) return rc;
    }
    return decode(pool, B, slot_ids, q, a_or_k, b_or_v, lambda, beta, out, stream, false, ptr, chunk);
}

int dl_decode_window(dl_pool *pool, int32_t B, const int32_t *slot_ids, int32_t W, const void *q,
                     const void *a_or_k, const void *b_or_v, const float *lambda, const float *beta, float *out,
                     void *stream) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    const dl_pool_desc &d = pool->desc;
    if (W < 1 || W > dl::kMaxWindow)
        return fail(DL_ERR_INVALID_ARG, "window length must be in [1, %d] (got %d)", dl::kMaxWindow, W);
    int rc = check_slots(pool, B, slot_ids);
    if (rc) return rc;
    if (d.decay == DL_DECAY_NONE && lambda) return fail(DL_ERR_INVALID_ARG, "lambda must be NULL for DL_DECAY_NONE");
    if (d.update == DL_UPDATE_PLAIN && beta) return fail(DL_ERR_INVALID_ARG, "beta must be NULL for DL_UPDATE_PLAIN");
    if (B == 0) return ok();
    if (!pool->dry) {
        if (!q || !a_or_k || !b_or_v || !out) return fail(DL_ERR_INVALID_ARG, "NULL q / a_or_k / b_or_v / out");
        if (d.decay != DL_DECAY_NONE && !lambda) return fail(DL_ERR_INVALID_ARG, "lambda is NULL");
        if (d.update == DL_UPDATE_DELTA && !beta) return fail(DL_ERR_INVALID_ARG, "beta is NULL");
        const uintptr_t align = (uintptr_t)q | (uintptr_t)a_or_k | (uintptr_t)b_or_v | (uintptr_t)out;
        if (align & 15) return fail(DL_ERR_INVALID_ARG, "token buffers must be 16-byte aligned");
        const int C = d.merge_interval - 1;
        const size_t D = d.d_k, Hv = d.num_v_heads, Hk = d.num_k_heads, s_in = dtype_size(d.in_dtype);
        const size_t lam_w = d.decay == DL_DECAY_PER_KEY ? D : 1;
        const size_t shmem = dl::window_stage_bytes(d.d_k, pool->bv, C, d.decay, d.update, d.in_dtype);
        (void)capturing(pool, stream);
        dl::WindowParams p;
        memset(&p, 0, sizeof p);
        p.base = pool->buf.base;
        p.klog = pool->buf.klog;
        p.ulog = pool->buf.ulog;
        p.lamlog = pool->buf.lamlog;
        p.nlog = pool->buf.nlog;
        p.H_v = d.num_v_heads;
        p.H_k = d.num_k_heads;
        p.C = C;
        p.NV = pool->nv;
        p.W = W;
        p.B = B;
        auto launch = [&](int32_t lo, int32_t cnt) -> int {
            p.q = static_cast<const char *>(q) + (size_t)lo * Hk * D * s_in;
            p.k = static_cast<const char *>(a_or_k) + (size_t)lo * Hk * D * s_in;
            p.v = static_cast<const char *>(b_or_v) + (size_t)lo * Hv * D * s_in;
            p.lam = lambda ? lambda + (size_t)lo * Hv * lam_w : nullptr;
            p.beta = beta ? beta + (size_t)lo * Hv : nullptr;
            p.out = out + (size_t)lo * Hv * D;
            memcpy(p.slots, slot_ids + lo, cnt * sizeof(int32_t));
            p.nunits = cnt * d.num_v_heads * pool->nv;
            const int e = dl::launch_window(d.d_k, pool->bv, d.decay, d.update, d.state_dtype, d.in_dtype, p, shmem,
                                            (hipStream_t)stream);
            return e != hipSuccess ? hip_fail((hipError_t)e, "window kernel launch") : DL_OK;
        };
        // the window leaves every log it covers empty
        auto commit = [&](int32_t lo, int32_t cnt) { dl::mirror_clear(pool->n.data(), slot_ids + lo, cnt); };
        rc = dl::launch_chunks(B, dl::kMaxLaunchSlots, launch, commit);
        return rc ? rc : ok();
    }
    dl::mirror_clear(pool->n.data(), slot_ids, B);
    return ok();
}

int dl_merge(dl_pool *pool, int32_t n, const int32_t *slot_ids, void *stream) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    int rc = check_slots(pool, n, slot_ids);
    if (rc) return rc;
    if (n == 0) return ok();
    return merge_slots(pool, n, slot_ids, stream);
}

int dl_flush_all(dl_pool *pool, void *stream) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    // The mirror picks the slots with a live log while it follows the device;
    // once a call has been recorded into a graph (or this one would be), the
    // device counters may hold entries the mirror does not show, so every
    // slot is launched and each block merges what its counter holds.
    const bool all = capturing(pool, stream) || pool->stale;
    std::vector<int32_t> live;
    for (int32_t s = 0; s < pool->desc.num_slots; ++s)
        if (all || pool->n[s] > 0) live.push_back(s);
    if (live.empty()) return ok();
    return merge_slots(pool, (int32_t)live.size(), live.data(), stream);
}

int dl_get_log_len(const dl_pool *pool, int32_t *n_out) {
    if (!pool || !n_out) return fail(DL_ERR_INVALID_ARG, "NULL argument");
    memcpy(n_out, pool->n.data(), pool->n.size() * sizeof(int32_t));
    return ok();
}

int dl_schedule(const dl_pool *pool, int32_t B, const int32_t *slot_ids, int32_t *merge_out, int32_t *index_out) {
    if (!pool) return fail(DL_ERR_INVALID_ARG, "pool is NULL");
    if (B > 0 && (!merge_out || !index_out)) return fail(DL_ERR_INVALID_ARG, "NULL output array");
    int rc = check_slots(const_cast<dl_pool *>(pool), B, slot_ids);
    if (rc) return rc;
    const int32_t C = pool->desc.merge_interval - 1;
    for (int32_t j = 0; j < B; ++j) {
        const int32_t n = pool->n[slot_ids[j]];
        merge_out[j] = n == C ? 1 : 0;
        index_out[j] = n;
    }
    return ok();
}

int dl_read_log_len_device(dl_pool *pool, int32_t *n_out, void *stream) {
    if (!pool || !n_out) return fail(DL_ERR_INVALID_ARG, "NULL argument");
    if (pool->dry) return fail(DL_ERR_DRY_RUN, "host-only pool has no device counters");
    const size_t bytes = (size_t)pool->desc.num_slots * pool->desc.num_v_heads * pool->nv * sizeof(int32_t);
    hipError_t e = hipMemcpyAsync(n_out, pool->buf.nlog, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "reading log lengths");
    return ok();
}

int dl_value_tile(const dl_pool_desc *desc) {
    int rc = validate_desc(desc);
    if (rc) return rc;
    g_err.clear();
    return value_tile_of(desc);
}

const char *dl_last_error(void) { return g_err.c_str(); }

int32_t dl_launch_slot_limit(void) { return dl::kMaxLaunchSlots; }

}  // extern "C"
