// DeltaLog decode-step kernels for CDNA4 (gfx950).
//
// Sources: [DL] "DeltaLog: Deferred Materialization of Recurrent States for
// Linear Attention Decoding" -- Eq. 3, the append-merge cycle and logical-state
// equation of the design section, and the GPU-execution section (ReplayPrep,
// AppendDecode, Finalize, Merge); [FPGA] "A Persistent-State Dataflow
// Accelerator for Memory-Bound Linear Attention Decode on FPGA" -- grouped
// value heads.
//
// One block owns the d_k x B_V value tile of one (slot, v-head) pair.  Each
// block computes the key-side replay coefficients of its slot-head itself (the
// paper's ReplayPrep, fused) and owns its own live-length counter (Finalize),
// so nothing is shared between blocks within a launch except the key entry
// and decay snapshot, which only the first tile writes (the designated
// writer).  Per block:
//
//   1. the live length n: the host's value for the slot in a direct launch,
//      checked against the device counter (restaged when they differ); the
//      counter itself in a launch recorded into a graph.  Then every load is
//      issued before any is consumed: token inputs, the live log as 16-byte
//      chunks, then the base tile (RPT x 16-byte non-temporal loads per
//      thread over one contiguous run; the base is value-tile major)
//   2. l' = l_bar + lambda (l_bar = newest snapshot, or 0 for an empty log);
//      q~ = e^{l'} * q and k~ = e^{l'} * k go to LDS, the log lands in LDS as
//      stored
//   3. replay coefficients per live entry i (TPE threads per entry, DPP sums):
//      c^q_i = sum_r e^{l'_r - Lam_ir} K_ir q_r, c^k_i likewise with k, and
//      for a merge the decayed keys e^{l' - Lam_i} * K_i.  With a scalar or
//      no decay the raw sums K_i . q and K_i . k are instead formed in step 2,
//      as each key chunk is staged, and weighted e^{l' - Lam_i} where read
//   4. y_q = S_bar^T q~ + sum_i c^q_i U_i and y_k = S_bar^T k~ + sum_i c^k_i U_i:
//      per-thread FMAs over its rows, DPP / row-swap sums across the row
//      groups of a wave, an LDS sum across waves
//   5. per column: b = beta (v - y_k) (delta) or the given b; o = y_q + (a.q) b
//   6. append: U[n] <- b, K[n] <- a (the first v-head of a q/k group owns the
//      shared key entry), Lam[n] <- l', n <- n + 1
//      merge:  S_bar <- e^{l'} * S_bar + sum_i (e^{l'-Lam_i} K_i) U_i^T + a b^T
//      from the tile still in registers, n <- 0
//
// The eager baseline is the same block with no log: always step 6's merge
// branch with n = 0, i.e. read S, decay, correct, add the outer product, write
// S.  The standalone merge uses the same code with no token (lambda = 0).
// Split replay (a pool option) moves step 3 of appending slot-heads into a
// ReplayPrep kernel that runs once per (slot, v-head) and leaves the
// coefficients in a scratch buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dl_internal.hpp"

namespace dl {

typedef uint16_t bf16_t;   // IEEE bfloat16 bit pattern

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    // round to nearest, ties to even (finite inputs)
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Unpack a 16-byte register vector of T into fp32.
template <typename T, int N>
__device__ __forceinline__ void unpack_f32(const uint4 &w, float (&out)[N]) {
    static_assert(N * sizeof(T) == 16, "one 16-byte vector");
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 4) {
            out[j] = __uint_as_float(ws[j]);
        } else {
            out[2 * j] = __uint_as_float(ws[j] << 16);
            out[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
        }
    }
}

// Dot product of two 16-byte vectors of T, in fp32.
template <typename T>
__device__ __forceinline__ float dot16(const uint4 &a, const uint4 &b) {
    constexpr int N = 16 / (int)sizeof(T);
    float x[N], y[N];
    unpack_f32<T, N>(a, x);
    unpack_f32<T, N>(b, y);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) s += x[j] * y[j];
    return s;
}

template <typename T, int N>
__device__ __forceinline__ uint4 pack_16(const float (&x)[N]) {
    static_assert(N * sizeof(T) == 16, "one 16-byte vector");
    uint32_t ws[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 4) {
            ws[j] = __float_as_uint(x[j]);
        } else {
            ws[j] = (uint32_t)from_f32<bf16_t>(x[2 * j]) | ((uint32_t)from_f32<bf16_t>(x[2 * j + 1]) << 16);
        }
    }
    return make_uint4(ws[0], ws[1], ws[2], ws[3]);
}

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// Row access of a tile: byte base plus a 32-bit per-lane byte offset.  The
// base tile is read once per step and not again until the next step, so its
// loads carry the non-temporal (streaming) hint: they do not displace the
// live log and token data from the caches.
__device__ __forceinline__ uint4 ld16(const void *base, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(
        reinterpret_cast<const v4u32 *>(static_cast<const char *>(base) + off)));
}

__device__ __forceinline__ void st16(void *base, uint32_t off, const uint4 &v) {
    *reinterpret_cast<uint4 *>(static_cast<char *>(base) + off) = v;
}

// Stores of data no block reads again in this launch (the step's output and
// appended value factor) carry the non-temporal hint as well.
__device__ __forceinline__ void st16_stream(void *base, uint32_t off, const uint4 &v) {
    __builtin_nontemporal_store(__builtin_bit_cast(v4u32, v), reinterpret_cast<v4u32 *>(static_cast<char *>(base) + off));
}

// ---- cross-lane sums in the vector ALU (no LDS round trip): DPP moves within
// a 16-lane row, and the gfx950 row swaps across rows.  All lanes of the wave
// must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- 7 - i within each 8
constexpr int kDppRowMirror = 0x140;      // lane i <- 15 - i within each row
constexpr int kDppRowRor = 0x120;         // + n: lane i <- (i + n) mod 16 within each row

// x of lane i plus x of lane i ^ 16 (rows 0 <-> 1, 2 <-> 3): the swap hands
// back both halves, whose sum is the row-pair sum in every lane.
__device__ __forceinline__ float sum_rows_xor1(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x of lane i plus x of lane i ^ 32
__device__ __forceinline__ float sum_rows_xor2(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64),
// returned in every lane of the group.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 2) x += dpp_f32<kDppQuadXor1>(x);
    if constexpr (W >= 4) x += dpp_f32<kDppQuadXor2>(x);
    if constexpr (W >= 8) x += dpp_f32<kDppRowHalfMirror>(x);   // the other quad of the 8
    if constexpr (W >= 16) x += dpp_f32<kDppRowMirror>(x);      // the other 8 of the row
    if constexpr (W >= 32) x = sum_rows_xor1(x);
    if constexpr (W >= 64) x = sum_rows_xor2(x);
    return x;
}

// Sum over the lanes of a wave that agree modulo S (S a power of two <= 64),
// returned in every lane: rotations by S, 2S, .. 8 close the ring of such
// lanes inside a row, then the rows are added.
template <int S>
__device__ __forceinline__ float strided_sum(float x) {
    if constexpr (S <= 1) x += dpp_f32<kDppRowRor + 1>(x);
    if constexpr (S <= 2) x += dpp_f32<kDppRowRor + 2>(x);
    if constexpr (S <= 4) x += dpp_f32<kDppRowRor + 4>(x);
    if constexpr (S <= 8) x += dpp_f32<kDppRowRor + 8>(x);
    if constexpr (S <= 16) x = sum_rows_xor1(x);
    if constexpr (S <= 32) x = sum_rows_xor2(x);
    return x;
}

// Blocks are dispatched round-robin over the 8 XCDs.  Renumber them so that
// each XCD works on a contiguous range of units: the value tiles and v-heads
// of one q/k group (which share the key-log entries and q / k) then meet in
// the same L2.
__device__ __forceinline__ int xcd_unit(int bid, int nb) {
    if ((nb & 7) != 0) return bid;
    return (bid & 7) * (nb >> 3) + (bid >> 3);
}
__device__ __forceinline__ uint32_t xcd_unit_u(uint32_t bid, uint32_t nb) {
    if ((nb & 7) != 0) return bid;
    return (bid & 7) * (nb >> 3) + (bid >> 3);
}

// q/k head of v-head h: h / (H_v / H_k) as the high word of 2h * gdiv, with
// gdiv = ceil(2^31 / (H_v / H_k)) from the host.  Exact while
// h * (gdiv * (H_v / H_k) - 2^31) < 2^31, which holds for H_v <= 32768 (the
// pool refuses more); gdiv = 2^31 gives h itself.  No branch, no division.
__device__ __forceinline__ uint32_t qk_head(uint32_t h, uint32_t gdiv) { return __umulhi(h + h, gdiv); }
// h is the first v-head of its q/k group (the group's key-factor writer):
// its q/k head differs from that of h - 1.  At h = 0 the unsigned 2h - 2
// wraps to 2^32 - 2, whose high word gdiv - 1 is not 0.
__device__ __forceinline__ bool first_of_group(uint32_t h, uint32_t gdiv) {
    return __umulhi(h + h, gdiv) != __umulhi(h + h - 2u, gdiv);
}

// Block geometry: a block owns the D x BV value tile of one (slot, v-head)
// ([DL] GPU-execution section: work units own d_k x B_V tiles, N_V = d_v / B_V).
template <int D, int BV, typename ST>
struct Tile {
    static constexpr int VEC = 16 / (int)sizeof(ST);       // elements per 16-byte load
    static constexpr int CG = BV / VEC;                    // column groups per tile row
    static constexpr int NT = D >= 128 ? 256 : (D >= 64 ? 128 : 64);
    static constexpr int RG = NT / CG;                     // row groups
    static constexpr int RPT = (D + RG - 1) / RG;          // rows per thread
    static constexpr int NW = NT / 64;                     // waves per block
    static constexpr bool RAGGED = RG > D;                 // some row groups own no row
    // keys per thread in the coefficient phase (measured: 8 for fp32 state
    // tiles, 4 for bf16 ones, whose unpacked tile leaves fewer free registers)
    static constexpr int KPT = sizeof(ST) == 2 ? 4 : 8;
    static constexpr int TPE = D / KPT;                    // threads per log entry
    static constexpr int EPP = NT / TPE;                   // log entries per coefficient pass
    // log chunks per thread loaded up front (longer logs stream in a loop);
    // 4 for bf16 tiles keeps their kernels, with the packed q / a of the
    // fused replay, within 128 VGPRs (4 waves per SIMD)
    static constexpr int PF = (RPT >= 16 || sizeof(ST) == 2) ? 4 : 8;
    static_assert(BV % VEC == 0 && D % BV == 0 && NT % CG == 0 && CG <= 64 && TPE <= 64 && NT >= D,
                  "tile geometry");
};

// N consecutive elements of type T from LDS, as fp32 (N a multiple of 4).
template <typename T, int N>
__device__ __forceinline__ void lds_f32(const T *src, float (&x)[N]) {
#pragma unroll
    for (int c = 0; c < N; c += 4) {
        if constexpr (sizeof(T) == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(src + c);
            x[c] = v.x;
            x[c + 1] = v.y;
            x[c + 2] = v.z;
            x[c + 3] = v.w;
        } else {
            const uint2 v = *reinterpret_cast<const uint2 *>(src + c);
            x[c] = __uint_as_float(v.x << 16);
            x[c + 1] = __uint_as_float(v.x & 0xffff0000u);
            x[c + 2] = __uint_as_float(v.y << 16);
            x[c + 3] = __uint_as_float(v.y & 0xffff0000u);
        }
    }
}

// Key-side replay coefficients of a slot-head's live log ([DL] Algorithm 1,
// ReplayPrep), TPE threads per entry with KPT keys each: the decayed key
// Kt_i = e^{l' - Lam_i} * K_i, c^q_i = Kt_i . q and c^k_i = Kt_i . k for i < n;
// the pass that reaches i == n computes a . q.  For a merge, Kt_i is kept in
// the snapshot slot (per-key decay) or the entry's scalar weight in s_w.
// Inputs in LDS: keys s_lk [n][D] as stored, snapshots s_ll [n][D] (per key)
// or s_lam [n] (scalar), l' in s_lp, q in s_qr, a (= k) in s_a.
template <int D, int NT, int KPT, int DECAY, bool DELTA, bool TOKEN, typename IT>
__device__ __forceinline__ void replay_coefficients(int tid, int n, bool merge, const IT *s_lk, float *s_ll,
                                                    const float *s_lp, const float *s_lam, const float *s_qr,
                                                    const float *s_a, float *s_cq, float *s_ck, float *s_w,
                                                    float &s_s) {
    constexpr int TPE = D / KPT;                 // threads per log entry
    constexpr int EPP = NT / TPE;                // log entries per pass
    constexpr bool PERKEY = DECAY == DECAY_PER_KEY;
    constexpr bool SCALAR = DECAY == DECAY_SCALAR;
    for (int i0 = 0; i0 <= n; i0 += EPP) {
        const int i = i0 + tid / TPE;
        const int r0 = (tid % TPE) * KPT;
        float pq = 0.f, pk = 0.f;
        if (i < n) {
            const float w = SCALAR ? __expf(s_lp[0] - s_lam[i]) : 1.f;
            if (!PERKEY && merge && r0 == 0) s_w[i] = w;
#pragma unroll
            for (int q4 = r0; q4 < r0 + KPT; q4 += 4) {
                float kt[4];
                lds_f32<IT, 4>(s_lk + i * D + q4, kt);
                if constexpr (PERKEY) {
                    const float4 l4 = *reinterpret_cast<const float4 *>(s_ll + i * D + q4);
                    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) kt[j] *= __expf(s_lp[q4 + j] - lv[j]);
                    // the snapshot is not read again: a merge keeps the decayed key there
                    if (merge) *reinterpret_cast<float4 *>(s_ll + i * D + q4) = make_float4(kt[0], kt[1], kt[2], kt[3]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) kt[j] *= w;
                }
                if constexpr (TOKEN) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pq += kt[j] * s_qr[q4 + j];
                        if constexpr (DELTA) pk += kt[j] * s_a[q4 + j];
                    }
                }
            }
        } else if (TOKEN && i == n) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) pq += s_a[r0 + j] * s_qr[r0 + j];
        }
        if constexpr (TOKEN) {
            pq = group_sum<TPE>(pq);
            if constexpr (DELTA) pk = group_sum<TPE>(pk);
            if (tid % TPE == 0) {
                if (i < n) {
                    s_cq[i] = pq;
                    s_ck[i] = pk;
                } else if (i == n) {
                    s_s = pq;
                }
            }
        }
    }
}

template <int D, int BV, int DECAY, bool DELTA, typename ST, typename IT, int MODE>
__global__ void __launch_bounds__((Tile<D, BV, ST>::NT))
dl_step_kernel(const int32_t H_v, const int32_t H_k, const int32_t C, const uint32_t gdiv, const uint32_t slot0,
               void *const base, int32_t *const nlog, const StepParams p) {
    using G = Tile<D, BV, ST>;
    using BT = typename std::conditional<DELTA, float, IT>::type;   // value-factor storage
    constexpr int NT = G::NT, VEC = G::VEC, CG = G::CG, RG = G::RG, RPT = G::RPT, NW = G::NW;
    constexpr int KPT = G::KPT, PF = G::PF;
    constexpr int NV = D / BV;                    // value tiles per slot-head
    constexpr int KV = 16 / (int)sizeof(IT);      // key-factor elements per 16-byte chunk
    constexpr int UV = 16 / (int)sizeof(BT);      // value-factor elements per 16-byte chunk
    constexpr int UCH = BV / UV;                  // value-factor chunks per entry and tile
    constexpr bool TOKEN = MODE != MODE_MERGE;
    constexpr bool LOG = MODE != MODE_EAGER;
    constexpr bool SPLIT = MODE == MODE_STEP_SPLIT;   // appends read ReplayPrep's coefficients
    constexpr bool CONSEC = MODE == MODE_STEP_CONSEC; // slots slot0 + e, live lengths from the device
    constexpr bool STEP = MODE == MODE_STEP || SPLIT || CONSEC;
    constexpr bool HINTED = MODE == MODE_STEP || CONSEC;  // loads follow the host's live length, if given
    // Scalar or no decay: the replay coefficients' raw dot products are formed
    // while the log is staged (one key chunk per thread, DPP sums over the
    // chunk's CPE threads) and weighted e^{l'-Lam_i} where they are read, so
    // there is no separate coefficient pass or barrier.  Per-key decay needs
    // the snapshot chunk beside each key chunk and keeps the pass.
    constexpr bool FC = (MODE == MODE_STEP || CONSEC || MODE == MODE_EAGER) && DECAY != DECAY_PER_KEY;
    constexpr int CPE = D / (16 / (int)sizeof(IT));   // 16-byte key chunks per log entry
    constexpr bool PERKEY = DECAY == DECAY_PER_KEY;
    constexpr bool SCALAR = DECAY == DECAY_SCALAR;
    // Narrow tiles (B_V <= 32: small batches) of a decode launch with scalar or
    // no decay stage the log by entries: a lane takes two adjacent key chunks
    // of one entry, so an entry spans TPE2 = CPE / 2 lanes and one round of
    // the block covers EPR entries (16 at d = 128 with fp32 keys), while the
    // value-factor chunks go to lanes of their own.  Against chunk rounds over
    // the whole log this halves the lanes each replay dot product is summed
    // over, needs one round for a log of up to EPR entries, and leaves no lane
    // choosing between log arrays.  Each lane's instructions count at batch 1,
    // where a block has its CU to itself and a wave issues one instruction
    // per four cycles.
    constexpr bool SMALL = HINTED && FC && BV <= 32 && CPE >= 2;
    constexpr int TPE2 = SMALL ? CPE / 2 : 1;         // lanes per log entry (narrow tiles)
    constexpr int EPR = NT / TPE2;                    // log entries per round (narrow tiles)
    constexpr int QP = SMALL ? 2 : 1;                 // key chunks of q and a per lane
    static_assert(BV % UV == 0, "value-factor chunks");

    __shared__ float s_q[D];        // e^{l'} * q
    __shared__ float s_k[D];        // e^{l'} * k
    __shared__ float s_qr[D];       // q
    __shared__ float s_a[D];        // a (= k for delta)
    __shared__ float s_g[D];        // e^{l'}
    __shared__ float s_lp[D];       // l'
    __shared__ __align__(16) float s_b[BV];   // b on this tile's columns (merge broadcast)
    __shared__ __align__(16) float s_v[BV];   // v on this tile's columns
    __shared__ float s_cq[kMaxLogCap + 1];
    __shared__ float s_ck[kMaxLogCap + 1];
    __shared__ float s_lam[kMaxLogCap + 1];   // scalar snapshots
    __shared__ float s_w[kMaxLogCap + 1];     // e^{l' - Lam_i} of a scalar decay (merge)
    __shared__ __align__(16) float s_red[NW][2][BV];
    __shared__ float s_s;           // a . q
    extern __shared__ float4 s_dyn[];

    // The launch geometry comes as leading scalar arguments (head counts, log
    // capacity, the q/k-head multiplier), which the build preloads into registers
    // before the block starts, so the block's slot word can be fetched at
    // once.  So do the first slot of a launch of consecutive slots, the base
    // and the live-length counters: such a block knows its slot and issues
    // its counter load before any argument has been fetched from memory.  The grid has one row per batch entry (blockIdx.y); along x run
    // the entry's (v-head, value tile) units, numbered so that each XCD holds
    // a contiguous run of them.  No integer division: a wave issues one
    // instruction per four cycles, and a division by a run-time value costs
    // about 25 of them ahead of the first load.  The q/k head of v-head h is
    // h / (H_v / H_k), from a host-computed multiplier (qk_head).
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ux = xcd_unit(blockIdx.x, H_v * NV);
    const int e = blockIdx.y;                           // batch entry of this launch
    const int h = ux / NV, vt = ux - h * NV;            // v-head, value tile
    const int eh = e * H_v + h;                         // (entry, v-head)
    const int c0 = vt * BV;                             // first column of the tile
    const int g = (int)qk_head((uint32_t)h, gdiv);
    // the first v-head of its q/k group writes the group's key factor
    const bool kwriter = first_of_group((uint32_t)h, gdiv);
    // The slot word: computed in a launch of consecutive slots (which carries
    // no live lengths from the host: the counter decides), else fetched with
    // every other argument the block reads, in one batch: left to itself the
    // compiler loads each where first used and waits for it before the next,
    // a chain of round trips ahead of the first HBM access.
    uint32_t sword;
    if constexpr (CONSEC) {
        sword = (slot0 + (uint32_t)e) | (kNoHint << kSlotBits);
    } else {
        sword = p.slots[e];
        asm volatile("" ::"s"(p.klog), "s"(p.ulog), "s"(p.lamlog), "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.lam),
                     "s"(p.beta), "s"(p.out), "s"(p.coef), "s"(sword));
    }
    const uint32_t slot = sword & kSlotMask;
    // Slot-head and slot-(q/k head) indices.  The host keeps P * H_v * N_V
    // below 2^31, so they and the (slot-head, tile) index fit 32 bits, and
    // each 64-bit offset below comes from one 32 x 32-bit product.
    const uint32_t sh32 = slot * (uint32_t)H_v + (uint32_t)h;
    const uint32_t gk32 = slot * (uint32_t)H_k + (uint32_t)g;
    const uint32_t shv = sh32 * NV + (uint32_t)vt;      // (slot-head, value tile): counter, base tile
    const size_t shC = (size_t)sh32 * (uint32_t)C;      // its first log entry
    const size_t gkC = (size_t)gk32 * (uint32_t)C;      // the q/k head's first key-log entry
    const uint32_t ek = (uint32_t)e * H_k + g;          // token row of q, k
    const uint32_t ev = (uint32_t)eh;                   // token row of v, lambda, beta, output
    const int cg = tid % CG, rg = tid / CG;
    const bool owner = vt == 0;                         // writes the tile-shared log metadata

    // Live length n.  A direct decode launch takes the host's value for the
    // slot (the slot word's top byte), so that no load below waits for the
    // device counter; the counter, read alongside, decides (step 2 stages
    // again when the two differ, as after direct launches that follow a
    // graph capture).  A launch recorded into a graph carries no value and
    // waits for the counter, whose round trip the token loads below overlap.
    // The counter is a scalar load (its index is uniform and nothing has been
    // stored yet): the scalar path answers in about half the time of a vector
    // load, and its wait does not hold the token loads, which a vector load's
    // in-order count would.  The scalar cache starts every launch empty, so it
    // sees the previous launch's store.  A consecutive launch's block issues
    // it before any argument has arrived (its slot, the counter and base
    // pointers are in registers from the start), with the argument batch.
    int n_dev = 0;
    if constexpr (HINTED) n_dev = ((const __attribute__((address_space(4))) int32_t *)(size_t)nlog)[shv];
    if constexpr (CONSEC) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::"s"(p.klog), "s"(p.ulog), "s"(p.lamlog), "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.lam),
                     "s"(p.beta), "s"(p.out), "s"(p.coef));
    }

    // ---- 1. every load of the block is issued before any is consumed: the
    //         token inputs (while the counter is in flight), the whole live
    //         log, then the base tile.  Every lane issues the token loads
    //         alike (indices taken modulo d, values used by the lanes below
    //         d).  Under a branch, the 16-bit inputs' widening to fp32 made the
    //         compiler wait for them at the branch's end, a whole memory round
    //         trip before the log and tile loads were issued; and in
    //         narrow-tile launches the in-order wait counts stay exact, so the
    //         wait for the snapshots below lets the later loads stay in flight.
    float qv = 0.f, kv = 0.f, vv = 0.f, lam = 0.f, lbar = 0.f, beta = 0.f, lam_i = 0.f;
    float lp0 = 0.f;                                    // l' (narrow tiles with a scalar decay: every lane)
    IT qraw{}, kraw{}, vraw{};                          // as stored; widened after the tile loads
    auto token_loads = [&]() {
        const uint32_t qo = ek * D + (tid % D);
        qraw = reinterpret_cast<const IT *>(p.q)[qo];
        kraw = reinterpret_cast<const IT *>(p.k)[qo];
        vraw = reinterpret_cast<const IT *>(p.v)[ev * D + c0 + (tid % BV)];
        if constexpr (SCALAR) lam = p.lam[ev];
        if constexpr (PERKEY) lam = p.lam[ev * D + (tid % D)];
        if constexpr (DELTA) beta = p.beta[ev];
    };
    if constexpr (TOKEN) token_loads();
    const IT *klog = reinterpret_cast<const IT *>(p.klog);
    const BT *ulog = reinterpret_cast<const BT *>(p.ulog);
    const float *lamlog = p.lamlog;
    const uint4 *kb = reinterpret_cast<const uint4 *>(klog + gkC * D);
    const BT *ub = ulog + shC * D + c0;
    const uint4 *lb = reinterpret_cast<const uint4 *>(lamlog + shC * D);

    // Narrow tiles: every snapshot (scalar decay) and the first round of key
    // entries and of value-factor chunks are loaded for the log's whole
    // capacity while the counter is in flight, and only the live entries are
    // staged once it has landed: at small batch the stale entries cost no
    // time, and the log does not wait a round trip behind the counter.  Lane
    // i of every wave holds snapshot i.  (Decode launches have C >= 1: a pool
    // with L = 1 decodes with the eager kernel, and the launcher refuses
    // otherwise.)
    constexpr int RK = SMALL ? 2 : 1;                   // key rounds loaded up front (longer logs stream)
    constexpr int RU = SMALL ? 2 : 1;                   // value-factor rounds loaded up front
    uint4 pk[RK][2], pu[RU];
    float lam_w = 0.f, pl[RK] = {};                     // snapshots: of lane i's entry i / of the lane's key entry
    if constexpr (SMALL && SCALAR) {
        lam_w = lamlog[shC + min(lane, C - 1)];
        pl[0] = lamlog[shC + min(tid / TPE2, C - 1)];
    }
    // q and a on the keys of this thread's key chunks (the same positions for
    // every chunk it stages), kept packed until used
    uint4 qpk[QP], apk[QP];
#pragma unroll
    for (int c = 0; c < QP; ++c) qpk[c] = apk[c] = make_uint4(0, 0, 0, 0);
    if constexpr (FC && TOKEN) {
        const int kc = SMALL ? (tid % TPE2) * 2 : tid % CPE;    // first key chunk of the lane
        const uint32_t qo = ek * D + kc * KV;
#pragma unroll
        for (int c = 0; c < QP; ++c) {
            qpk[c] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const IT *>(p.q) + qo + c * KV);
            apk[c] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const IT *>(p.k) + qo + c * KV);
        }
    }
    if constexpr (SMALL) {
        const uint4 *src = kb + (size_t)min(tid / TPE2, C - 1) * CPE + (tid % TPE2) * 2;
        pk[0][0] = src[0];
        pk[0][1] = src[1];
        const int u = min(tid, C * UCH - 1), j = u / UCH;
        pu[0] = *reinterpret_cast<const uint4 *>(ub + (size_t)j * D + (u - j * UCH) * UV);
    }

    int n = 0;
    if constexpr (HINTED) {
        const uint32_t hint = sword >> kSlotBits;
        n = hint == kNoHint ? min(max(__builtin_amdgcn_readfirstlane(n_dev), 0), C) : min((int)hint, C);
    } else if constexpr (LOG) {
        n = nlog[shv];
    }
    if constexpr (MODE == MODE_MERGE) {
        if (n == 0) return;                             // empty log: nothing to materialize
    }
    bool merge = !STEP || (n == C);
    const bool fused = !SPLIT || merge;                 // this block replays its own coefficients

    if constexpr (!(SMALL && SCALAR)) {
        if constexpr (LOG) {
            if (tid < D && n > 0) {
                if constexpr (SCALAR) lbar = lamlog[shC + (n - 1)];
                if constexpr (PERKEY) lbar = lamlog[(shC + (n - 1)) * D + tid];
            }
        }
        if constexpr (SCALAR && LOG) {
            if (fused && tid < n) lam_i = lamlog[shC + tid];
        }
    }
    // split replay: this append's coefficients from the scratch (c^q, c^k per
    // live entry, then a . q)
    float cq_r = 0.f, ck_r = 0.f, s_r = 0.f;
    if constexpr (SPLIT) {
        if (!fused) {
            const float *cf = p.coef + (size_t)eh * (2 * (C + 1));
            if (tid < n) {
                cq_r = cf[tid];
                ck_r = cf[C + tid];
            }
            if (tid == n) s_r = cf[2 * C];
        }
    }
    // live log as 16-byte chunks: K entries of the shared q/k head (all D keys),
    // U entries on this tile's columns, per-key snapshots (all D keys)
    // the live log lands in LDS as stored, chunk x at byte 16 x: key factors
    // [n][D], value factors on this tile [n][BV], per-key snapshots [n][D]
    // (overwritten by e^{l'-Lam_i} * K_i for a merge)
    char *s_log = reinterpret_cast<char *>(s_dyn);
    const IT *s_lk = reinterpret_cast<const IT *>(s_log);
    int cK = 0, cU = 0, ctot = 0;
    const BT *s_lu = nullptr;
    float *s_ll = nullptr;
    auto log_layout = [&]() {
        cK = (LOG && fused) ? n * D / KV : 0;
        cU = LOG ? n * UCH : 0;
        const int cL = (LOG && PERKEY && fused) ? n * D / 4 : 0;
        ctot = cK + cU + cL;
        s_lu = reinterpret_cast<const BT *>(s_log + (size_t)cK * 16);
        s_ll = reinterpret_cast<float *>(s_log + (size_t)(cK + cU) * 16);
    };
    log_layout();
    auto chunk_ptr = [&](int x) -> const uint4 * {
        if (x < cK) return kb + x;
        if (x < cK + cU) {
            const int u = x - cK, i = u / UCH;
            return reinterpret_cast<const uint4 *>(ub + (size_t)i * D + (u - i * UCH) * UV);
        }
        return lb + (x - cK - cU);
    };
    // (stored per component: an aggregate copy out of the prefetch array would
    // keep that array in scratch memory)
    auto stage = [&](int x, const uint4 w) {
        *reinterpret_cast<uint4 *>(s_log + (size_t)x * 16) = make_uint4(w.x, w.y, w.z, w.w);
    };
    // raw replay dot products of key chunk x (entry x / CPE) with q and a,
    // completed over the entry's CPE consecutive threads; every thread of the
    // block calls this for the same chunk block
    auto chunk_dots = [&](const int x, const uint4 w) {
        float pq = 0.f, pk = 0.f;
        if (x < cK) {
            pq = dot16<IT>(w, qpk[0]);
            if constexpr (DELTA) pk = dot16<IT>(w, apk[0]);
        }
        pq = group_sum<CPE>(pq);
        if constexpr (DELTA) pk = group_sum<CPE>(pk);
        if (x < cK && x % CPE == 0) {
            s_cq[x / CPE] = pq;
            if constexpr (DELTA) s_ck[x / CPE] = pk;
        }
    };
    // narrow tiles: round r of key entries (entry r EPR + tid / TPE2, two
    // chunks per lane), staged with their raw dot products; value-factor
    // chunks u = r NT + tid
    // (with a scalar decay, each lane also holds its entry's snapshot and the
    // coefficients leave weighted by e^{l'-Lam_i}; the weight is kept for a
    // merge.  The keys reach LDS only for a merge, the one reader of them.)
    auto k_load = [&](const int r, uint4 (&w)[2], float &le) {
        const int i = r * EPR + tid / TPE2;
        if (i < n) {
            const uint4 *src = kb + (size_t)i * CPE + (tid % TPE2) * 2;
            w[0] = src[0];
            w[1] = src[1];
            if constexpr (SCALAR) le = lamlog[shC + i];
        }
    };
    auto k_stage = [&](const int r, const uint4 (&w)[2], const float le) {   // every lane, uniform r (DPP sums)
        const int i = r * EPR + tid / TPE2;
        float pq = 0.f, pk = 0.f;
        if (i < n) {
            if (merge) {
                const int x = i * CPE + (tid % TPE2) * 2;
                stage(x, w[0]);
                stage(x + 1, w[1]);
            }
            pq = dot16<IT>(w[0], qpk[0]) + dot16<IT>(w[1], qpk[QP - 1]);
            if constexpr (DELTA) pk = dot16<IT>(w[0], apk[0]) + dot16<IT>(w[1], apk[QP - 1]);
        }
        pq = group_sum<TPE2>(pq);
        if constexpr (DELTA) pk = group_sum<TPE2>(pk);
        if (i < n && tid % TPE2 == 0) {
            const float wt = SCALAR ? __expf(lp0 - le) : 1.f;
            s_cq[i] = pq * wt;
            if constexpr (DELTA) s_ck[i] = pk * wt;
            if (merge) s_w[i] = wt;
        }
    };
    auto u_load = [&](const int r, uint4 &w) {
        const int u = r * NT + tid;
        if (u < cU) {
            const int i = u / UCH;
            w = *reinterpret_cast<const uint4 *>(ub + (size_t)i * D + (u - i * UCH) * UV);
        }
    };
    auto u_stage = [&](const int r, const uint4 &w) {
        const int u = r * NT + tid;
        if (u < cU) stage(cK + u, w);
    };
    // (the chunk rounds past the live log are left by a uniform branch: a
    // short log pays for the rounds it uses, not for the capacity's)
    uint4 pf[PF];
    if constexpr (SMALL) {                              // round 0 is in flight already
#pragma unroll
        for (int r = 1; r < RK; ++r) {
            if (r * EPR >= n) break;
            k_load(r, pk[r], pl[r]);
        }
#pragma unroll
        for (int r = 1; r < RU; ++r) {
            if (r * NT >= cU) break;
            u_load(r, pu[r]);
        }
    } else if constexpr (LOG) {
#pragma unroll
        for (int m = 0; m < PF; ++m) {
            if (m * NT >= ctot) break;
            const int x = tid + m * NT;
            if (x < ctot) pf[m] = *chunk_ptr(x);
        }
    }
    // base tile, issued after the log so that the coefficient phase below
    // overlaps its arrival.  The base is value-tile major, [slot-head][NV][D][BV],
    // so the tile is one contiguous run: a thread reads tile rows rg + RG * j,
    // columns cg * VEC ..
    const ST *tbase = reinterpret_cast<const ST *>(base) + (size_t)shv * (D * BV);
    const uint32_t toff = (uint32_t)((rg * BV + cg * VEC) * sizeof(ST));
    constexpr uint32_t TROW = RG * BV * sizeof(ST);     // bytes between a thread's rows
    uint4 tile[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        if (!G::RAGGED || rg + RG * j < D) tile[j] = ld16(tbase, toff + j * TROW);
        else tile[j] = make_uint4(0, 0, 0, 0);
    }
    // 16-bit token inputs are widened only now, behind a scheduling barrier
    // at d = 128: widened earlier, the compiler waited for them ahead of the
    // tile loads (KDA-style batch 128: 2% per step, the serving pool 1%).  At
    // d = 64 the barrier measured slower (GLA-style eager kernel 19%).
    if constexpr (TOKEN) {
        if constexpr (sizeof(IT) == 2 && D >= 128) __builtin_amdgcn_sched_barrier(0);
        qv = to_f32(qraw);
        kv = to_f32(kraw);
        vv = to_f32(vraw);
    }

    // ---- 2. decay bookkeeping, decayed q / k, and the log into LDS
    auto stage_decay = [&](const float lb) {            // rows tid < D
        const float lp = lb + lam;                      // l' = l_bar + lambda
        const float gg = (DECAY == DECAY_NONE) ? 1.f : __expf(lp);
        s_lp[tid] = lp;
        s_g[tid] = gg;
        if constexpr (TOKEN) {
            s_qr[tid] = qv;
            s_a[tid] = kv;
            s_q[tid] = gg * qv;
            s_k[tid] = gg * kv;
            if (tid < BV) s_v[tid] = vv;
        }
    };
    if constexpr (SMALL && SCALAR)                      // snapshot n - 1 from lane n - 1 (uniform n)
        lbar = n > 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_w), n - 1)) : 0.f;
    lp0 = lbar + lam;
    if (tid < D) stage_decay(lbar);
    if constexpr (LOG) {
        if constexpr (SCALAR) {
            if (!SMALL && fused && tid < n) s_lam[tid] = lam_i;
        }
        if constexpr (SPLIT) {
            if (!fused) {
                if (tid < n) {
                    s_cq[tid] = cq_r;
                    s_ck[tid] = ck_r;
                }
                if (tid == n) s_s = s_r;
            }
        }
        if constexpr (SMALL) {
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                if (r * EPR >= n) break;
                k_stage(r, pk[r], pl[r]);
            }
            for (int r = RK; r * EPR < n; ++r) {        // long logs
                uint4 w[2];
                float le = 0.f;
                k_load(r, w, le);
                k_stage(r, w, le);
            }
#pragma unroll
            for (int r = 0; r < RU; ++r) {
                if (r * NT >= cU) break;
                u_stage(r, pu[r]);
            }
            for (int r = RU; r * NT < cU; ++r) {
                uint4 w;
                u_load(r, w);
                u_stage(r, w);
            }
        } else {
#pragma unroll
        for (int m = 0; m < PF; ++m) {
            if (m * NT >= ctot) break;
            const int x = tid + m * NT;
            if (x < ctot) stage(x, pf[m]);
            if constexpr (FC && TOKEN) {
                if (m * NT < cK) chunk_dots(x, pf[m]);
            }
        }
        if constexpr (FC && TOKEN) {
            for (int xb = PF * NT; xb < ctot; xb += NT) {   // long logs (uniform trip count: DPP sums inside)
                const int x = xb + tid;
                uint4 w = make_uint4(0, 0, 0, 0);
                if (x < ctot) {
                    w = *chunk_ptr(x);
                    stage(x, w);
                }
                if (xb < cK) chunk_dots(x, w);
            }
        } else {
            for (int x = tid + PF * NT; x < ctot; x += NT) stage(x, *chunk_ptr(x));   // long logs
        }
        }
    }
    if constexpr (FC && TOKEN) {                        // a . q, summed by the first chunk group
        constexpr int AG = SMALL ? TPE2 : CPE;          // lanes holding the D keys
        float pa = 0.f;
        if (tid < AG) {
#pragma unroll
            for (int c = 0; c < QP; ++c) pa += dot16<IT>(qpk[c], apk[c]);
        }
        pa = group_sum<AG>(pa);
        if (tid == 0) s_s = pa;
    }
    if constexpr (HINTED) {
        const int nd = __builtin_amdgcn_readfirstlane(n_dev);
        if (nd != n) {                           // the host's value is stale: stage n_dev entries
            __syncthreads();                            // every speculative chunk has landed
            n = min(max(nd, 0), C);
            merge = n == C;
            log_layout();
            if constexpr (SMALL && SCALAR) {
                lbar = n > 0 ? lamlog[shC + (n - 1)] : 0.f;
                lp0 = lbar + lam;
                if (tid < D) stage_decay(lbar);
            } else {
                if (tid < D) {
                    float lb = 0.f;
                    if (n > 0) {
                        if constexpr (SCALAR) lb = lamlog[shC + (n - 1)];
                        if constexpr (PERKEY) lb = lamlog[(shC + (n - 1)) * D + tid];
                    }
                    stage_decay(lb);
                }
                if constexpr (SCALAR) {
                    if (tid < n) s_lam[tid] = lamlog[shC + tid];
                }
            }
            if constexpr (SMALL) {
                for (int r = 0; r * EPR < n; ++r) {
                    uint4 w[2];
                    float le = 0.f;
                    k_load(r, w, le);
                    k_stage(r, w, le);
                }
                for (int r = 0; r * NT < cU; ++r) {
                    uint4 w;
                    u_load(r, w);
                    u_stage(r, w);
                }
            } else if constexpr (FC && TOKEN) {
                for (int xb = 0; xb < ctot; xb += NT) {
                    const int x = xb + tid;
                    uint4 w = make_uint4(0, 0, 0, 0);
                    if (x < ctot) {
                        w = *chunk_ptr(x);
                        stage(x, w);
                    }
                    if (xb < cK) chunk_dots(x, w);
                }
            } else {
                for (int x = tid; x < ctot; x += NT) stage(x, *chunk_ptr(x));
            }
        }
    }
    __syncthreads();

    // ---- 3. replay coefficients: computed here, or (appending units of a
    //         split-replay launch) the ones ReplayPrep left in the scratch,
    //         loaded with the rest of the block's inputs
    if constexpr (!FC) {
        if (fused) {
            if constexpr (LOG)
                replay_coefficients<D, NT, KPT, DECAY, DELTA, TOKEN, IT>(tid, n, merge, s_lk, s_ll, s_lp, s_lam,
                                                                         s_qr, s_a, s_cq, s_ck, s_w, s_s);
            else
                replay_coefficients<D, NT, KPT, DECAY, DELTA, TOKEN, IT>(tid, 0, merge, s_lk, s_ll, s_lp, s_lam,
                                                                         s_qr, s_a, s_cq, s_ck, s_w, s_s);
        }
        __syncthreads();
    }

    // ---- 4-6. projections, value factor, output, append commit
    if constexpr (TOKEN) {
        float accq[VEC], acck[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) accq[c] = acck[c] = 0.f;
        if constexpr (LOG) {
            for (int i = rg; i < n; i += RG) {             // log entries as extra rows
                // staged raw dot products carry their decay weight here
                // (narrow tiles stage them weighted)
                const float wi = (FC && SCALAR && !SMALL) ? __expf(s_lp[0] - s_lam[i]) : 1.f;
                const float cq = s_cq[i] * wi, ck = s_ck[i] * wi;
                float u[VEC];
                lds_f32<BT, VEC>(s_lu + i * BV + cg * VEC, u);
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    accq[c] += cq * u[c];
                    if constexpr (DELTA) acck[c] += ck * u[c];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg + RG * j;
            if (!G::RAGGED || r < D) {
                float x[VEC];
                unpack_f32<ST, VEC>(tile[j], x);
                const float qr = s_q[r];
                const float kr = DELTA ? s_k[r] : 0.f;
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    accq[c] += x[c] * qr;
                    if constexpr (DELTA) acck[c] += x[c] * kr;
                }
            }
        }
        // row groups of a wave: lanes that agree modulo CG hold the same columns
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            accq[c] = strided_sum<CG>(accq[c]);
            if constexpr (DELTA) acck[c] = strided_sum<CG>(acck[c]);
        }
        if (lane < CG) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                s_red[wave][0][cg * VEC + c] = accq[c];
                s_red[wave][1][cg * VEC + c] = acck[c];
            }
        }
        // stores that need no reduced value go out before the barrier, once
        // this wave's loads are consumed: the appended token's tile-shared
        // entries (key factor from the first v-head of the q/k group, decay
        // snapshot; first tile only) and this block's live-length counter.
        // No block of this launch reads entry n or another block's counter.
        if constexpr (LOG) {
            if (!merge && owner && tid < D) {
                if (kwriter) reinterpret_cast<IT *>(p.klog)[(gkC + n) * D + tid] = kraw;
                if constexpr (PERKEY) p.lamlog[(shC + n) * D + tid] = s_lp[tid];
                if constexpr (SCALAR) {
                    if (tid == 0) p.lamlog[shC + n] = s_lp[0];
                }
            }
            if (tid == 0) nlog[shv] = merge ? 0 : n + 1;
        }
        __syncthreads();

        // output and appended value factor leave in one 16-byte store per lane:
        // NO lanes cover 4 output columns each, then NU lanes one value-factor
        // chunk (UV columns) each.  Out lanes also publish b for a merge.
        constexpr int NO = BV / 4;
        constexpr int NU = LOG ? BV / UV : 0;
        constexpr int MC = UV > 4 ? UV : 4;
        static_assert(NO + NU <= 64, "column lanes fit one wave");
        const bool is_u = tid >= NO;
        if (tid < NO || (tid < NO + NU && !merge)) {
            const int cb = is_u ? (tid - NO) * UV : tid * 4;       // first column in the tile
            const int nc = is_u ? UV : 4;
            float ov[MC], bc[MC];
#pragma unroll
            for (int c4 = 0; c4 < MC; c4 += 4) {
                if (c4 < nc) {
                    float4 yq = make_float4(0.f, 0.f, 0.f, 0.f), yk = yq;
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        const float4 a = *reinterpret_cast<const float4 *>(&s_red[w][0][cb + c4]);
                        yq.x += a.x; yq.y += a.y; yq.z += a.z; yq.w += a.w;
                        if constexpr (DELTA) {
                            const float4 b4 = *reinterpret_cast<const float4 *>(&s_red[w][1][cb + c4]);
                            yk.x += b4.x; yk.y += b4.y; yk.z += b4.z; yk.w += b4.w;
                        }
                    }
                    const float4 v4 = *reinterpret_cast<const float4 *>(&s_v[cb + c4]);
                    const float yqa[4] = {yq.x, yq.y, yq.z, yq.w}, yka[4] = {yk.x, yk.y, yk.z, yk.w};
                    const float va[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float b = DELTA ? beta * (va[j] - yka[j]) : va[j];
                        bc[c4 + j] = b;
                        ov[c4 + j] = yqa[j] + s_s * b;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bc[c4 + j] = ov[c4 + j] = 0.f;
                }
            }
            if (merge && !is_u)
                *reinterpret_cast<float4 *>(&s_b[cb]) = make_float4(bc[0], bc[1], bc[2], bc[3]);
            const uint4 wo = make_uint4(__float_as_uint(ov[0]), __float_as_uint(ov[1]),
                                        __float_as_uint(ov[2]), __float_as_uint(ov[3]));
            uint4 wu = wo;
            if constexpr (LOG) {
                float ub[UV];
#pragma unroll
                for (int c = 0; c < UV; ++c) ub[c] = bc[c];
                wu = pack_16<BT, UV>(ub);
            }
            char *dst = is_u ? reinterpret_cast<char *>(p.ulog) + ((shC + n) * D + c0 + cb) * sizeof(BT)
                             : reinterpret_cast<char *>(p.out) + ((size_t)ev * D + c0 + cb) * sizeof(float);
            // per-component select: a select of whole vectors goes through scratch
            st16_stream(dst, 0, make_uint4(is_u ? wu.x : wo.x, is_u ? wu.y : wo.y, is_u ? wu.z : wo.z,
                                    is_u ? wu.w : wo.w));
        }
    }
    if constexpr (MODE == MODE_MERGE) {
        if (tid == 0) nlog[shv] = 0;
    }
    if (!merge) return;

    // ---- merge: S_bar <- e^{l'} * S_bar + sum_i Kt_i U_i^T + a b^T on this tile, from registers
    __syncthreads();
    // 16-bit tiles: the packed tile is opaque from here, so the compiler cannot
    // widen it to fp32 ahead of the barrier, where the projection's registers
    // are still live (that would cost the whole-row kernels a wave per SIMD)
    if constexpr (sizeof(ST) == 2) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            v4u32 t = __builtin_bit_cast(v4u32, tile[j]);
            asm volatile("" : "+v"(t));
            tile[j] = __builtin_bit_cast(uint4, t);
        }
    }
    float acc[RPT][VEC];
    float bcol[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) bcol[c] = TOKEN ? s_b[cg * VEC + c] : 0.f;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = rg + RG * j;
        const int rr = r < D ? r : 0;
        unpack_f32<ST, VEC>(tile[j], acc[j]);
        const float gr = s_g[rr];
        const float ar = TOKEN ? s_a[rr] : 0.f;
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[j][c] = gr * acc[j][c] + ar * bcol[c];
    }
    if constexpr (LOG) {
        for (int i = 0; i < n; ++i) {
            float u[VEC];
            lds_f32<BT, VEC>(s_lu + i * BV + cg * VEC, u);
            const float w = PERKEY ? 0.f
                          : SMALL ? (SCALAR ? s_w[i] : 1.f)
                                  : (FC ? (SCALAR ? __expf(s_lp[0] - s_lam[i]) : 1.f) : s_w[i]);
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int r = rg + RG * j;
                const int rr = r < D ? r : 0;
                const float kt = PERKEY ? s_ll[i * D + rr] : to_f32(s_lk[i * D + rr]) * w;
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[j][c] += kt * u[c];
            }
        }
    }
    ST *basew = const_cast<ST *>(tbase);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        if (!G::RAGGED || rg + RG * j < D) st16(basew, toff + j * TROW, pack_16<ST, VEC>(acc[j]));
    }
}

// ReplayPrep ([DL] GPU-execution section): one block per (entry, v-head) of
// the launch computes the key-side coefficients of the slot-head's live log
// once and leaves them in the scratch, 2 (C + 1) floats per (entry, v-head):
// c^q_i, then c^k_i at offset C, then a . q at offset 2 C.  Slot-heads about to
// merge are skipped: their decode units replay in-block, since a merge needs
// the decayed keys row by row.  Same arithmetic as the fused path.
template <int D, int DECAY, bool DELTA, typename ST, typename IT>
__global__ void __launch_bounds__((Tile<D, D, ST>::NT))
dl_replay_prep_kernel(const StepParams p) {
    using G = Tile<D, D, ST>;
    constexpr int NT = G::NT, KPT = G::KPT;
    constexpr int KV = 16 / (int)sizeof(IT);
    constexpr int PF = 4;
    constexpr bool PERKEY = DECAY == DECAY_PER_KEY;
    constexpr bool SCALAR = DECAY == DECAY_SCALAR;

    __shared__ float s_lp[D];
    __shared__ float s_qr[D];
    __shared__ float s_a[D];
    __shared__ float s_cq[kMaxLogCap + 1];
    __shared__ float s_ck[kMaxLogCap + 1];
    __shared__ float s_lam[kMaxLogCap + 1];
    __shared__ float s_w[kMaxLogCap + 1];
    __shared__ float s_s;
    extern __shared__ float4 s_dyn[];

    const int tid = threadIdx.x;
    const int unit = blockIdx.x;                       // (entry, v-head) of this launch
    const int H_v = p.H_v, C = p.C;
    const int e = unit / H_v, h = unit - e * H_v;
    const int g = h / (H_v / p.H_k);
    const int slot = (int)(p.slots[e] & kSlotMask);
    const size_t sh = (size_t)slot * H_v + h;
    const size_t gk = (size_t)slot * p.H_k + g;
    const int n = p.nlog[sh * p.NV];                   // every tile of the slot-head holds the same
    if (n == C) return;

    float qv = 0.f, kv = 0.f, lam = 0.f, lbar = 0.f, lam_i = 0.f;
    if (tid < D) {
        const size_t qo = ((size_t)e * p.H_k + g) * D + tid;
        qv = to_f32(reinterpret_cast<const IT *>(p.q)[qo]);
        kv = to_f32(reinterpret_cast<const IT *>(p.k)[qo]);
        if constexpr (SCALAR) lam = p.lam[(size_t)e * H_v + h];
        if constexpr (PERKEY) lam = p.lam[((size_t)e * H_v + h) * D + tid];
        if (n > 0) {
            if constexpr (SCALAR) lbar = p.lamlog[sh * C + (n - 1)];
            if constexpr (PERKEY) lbar = p.lamlog[(sh * C + (n - 1)) * D + tid];
        }
    }
    if constexpr (SCALAR) {
        if (tid < n) lam_i = p.lamlog[sh * C + tid];
    }
    // key entries of the q/k head, then per-key snapshots, as stored, chunk x at byte 16 x
    const int cK = n * D / KV;
    const int ctot = cK + (PERKEY ? n * D / 4 : 0);
    char *s_log = reinterpret_cast<char *>(s_dyn);
    const IT *s_lk = reinterpret_cast<const IT *>(s_log);
    float *s_ll = reinterpret_cast<float *>(s_log + (size_t)cK * 16);
    const uint4 *kb = reinterpret_cast<const uint4 *>(reinterpret_cast<const IT *>(p.klog) + gk * C * D);
    const uint4 *lb = reinterpret_cast<const uint4 *>(p.lamlog + sh * C * D);
    auto chunk_ptr = [&](int x) -> const uint4 * { return x < cK ? kb + x : lb + (x - cK); };
    uint4 pf[PF];
#pragma unroll
    for (int m = 0; m < PF; ++m) {
        const int x = tid + m * NT;
        if (x < ctot) pf[m] = *chunk_ptr(x);
    }
    if (tid < D) {
        s_lp[tid] = lbar + lam;
        s_qr[tid] = qv;
        s_a[tid] = kv;
    }
    if constexpr (SCALAR) {
        if (tid < n) s_lam[tid] = lam_i;
    }
#pragma unroll
    for (int m = 0; m < PF; ++m) {
        const int x = tid + m * NT;
        if (x < ctot) {
            const uint4 w = pf[m];
            *reinterpret_cast<uint4 *>(s_log + (size_t)x * 16) = make_uint4(w.x, w.y, w.z, w.w);
        }
    }
    for (int x = tid + PF * NT; x < ctot; x += NT) {
        const uint4 w = *chunk_ptr(x);
        *reinterpret_cast<uint4 *>(s_log + (size_t)x * 16) = make_uint4(w.x, w.y, w.z, w.w);
    }
    __syncthreads();
    replay_coefficients<D, NT, KPT, DECAY, DELTA, true, IT>(tid, n, false, s_lk, s_ll, s_lp, s_lam, s_qr, s_a,
                                                             s_cq, s_ck, s_w, s_s);
    __syncthreads();
    float *cf = p.coef + (size_t)unit * (2 * (C + 1));
    for (int i = tid; i < n; i += NT) {
        cf[i] = s_cq[i];
        cf[C + i] = s_ck[i];
    }
    if (tid == 0) cf[2 * C] = s_s;
}

}  // namespace dl

#include "dl_small.hpp"

namespace dl {

template <int D, int BV, int DECAY, bool DELTA, typename ST, typename IT>
static hipError_t launch_combo(int mode, const StepParams &p, size_t shmem, hipStream_t s) {
    constexpr int NT = Tile<D, BV, ST>::NT;
    constexpr int NV = D / BV;
    const dim3 block(NT);
    if (mode == MODE_REPLAY_PREP) {
        dl_replay_prep_kernel<D, DECAY, DELTA, ST, IT><<<dim3(p.nunits), block, shmem, s>>>(p);
        return hipGetLastError();
    }
    // decode / eager / merge: one grid row per batch entry
    const int per_entry = p.H_v * NV;
    if (p.H_k <= 0 || p.H_v % p.H_k != 0 || p.nunits % per_entry != 0) return hipErrorInvalidValue;
    if (mode != MODE_EAGER && p.C < 1) return hipErrorInvalidValue;    // the log kernels need a log
    const dim3 grid(per_entry, p.nunits / per_entry);
    const uint32_t grp = (uint32_t)(p.H_v / p.H_k);
    if (p.H_v > 32768) return hipErrorInvalidValue;                   // qk_head exact below
    const uint32_t gdiv = (uint32_t)((0x80000000ull + grp - 1) / grp);
#define LEAD p.slot0, p.base, p.nlog
    // narrow tiles with a scalar or no decay: decode and eager steps run the
    // one-barrier kernel where its lane layout fits (at least 4 key chunks per
    // entry, every thread owning tile rows, at most 32 bytes of value factor
    // per lane)
    using BTn = typename std::conditional<DELTA, float, IT>::type;
    constexpr int CPEn = D / (16 / (int)sizeof(IT));
    constexpr bool NARROW = BV <= 32 && DECAY != DECAY_PER_KEY && CPEn >= 4 && !Tile<D, BV, ST>::RAGGED &&
                            (BV / (CPEn / 2)) * (int)sizeof(BTn) <= 32;
    switch (mode) {
    case MODE_STEP:
        if constexpr (NARROW)
            dl_small_kernel<D, BV, DECAY, DELTA, ST, IT, false><<<grid, block, shmem, s>>>(p.H_v, p.H_k, p.C, gdiv, p);
        else
            dl_step_kernel<D, BV, DECAY, DELTA, ST, IT, MODE_STEP><<<grid, block, shmem, s>>>(p.H_v, p.H_k, p.C, gdiv, LEAD, p);
        break;
    case MODE_EAGER:
        if constexpr (NARROW)
            dl_small_kernel<D, BV, DECAY, DELTA, ST, IT, true><<<grid, block, 0, s>>>(p.H_v, p.H_k, p.C, gdiv, p);
        else
            dl_step_kernel<D, BV, DECAY, DELTA, ST, IT, MODE_EAGER><<<grid, block, 0, s>>>(p.H_v, p.H_k, p.C, gdiv, LEAD, p);
        break;
    case MODE_MERGE:
        dl_step_kernel<D, BV, DECAY, DELTA, ST, IT, MODE_MERGE><<<grid, block, shmem, s>>>(p.H_v, p.H_k, p.C, gdiv, LEAD, p);
        break;
    case MODE_STEP_CONSEC:      // (narrow tiles read their slot words)
        if constexpr (NARROW)
            dl_small_kernel<D, BV, DECAY, DELTA, ST, IT, false><<<grid, block, shmem, s>>>(p.H_v, p.H_k, p.C, gdiv, p);
        else
            dl_step_kernel<D, BV, DECAY, DELTA, ST, IT, MODE_STEP_CONSEC><<<grid, block, shmem, s>>>(p.H_v, p.H_k, p.C, gdiv, LEAD, p);
        break;
    case MODE_STEP_SPLIT:
        dl_step_kernel<D, BV, DECAY, DELTA, ST, IT, MODE_STEP_SPLIT><<<grid, block, shmem, s>>>(p.H_v, p.H_k, p.C, gdiv, LEAD, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
#undef LEAD
}

template <int D, int BV, int DECAY, bool DELTA>
static hipError_t launch_dtypes(int mode, int st, int it, const StepParams &p, size_t shmem, hipStream_t s) {
    if (st == F32 && it == F32) return launch_combo<D, BV, DECAY, DELTA, float, float>(mode, p, shmem, s);
    if (st == F32 && it == BF16) return launch_combo<D, BV, DECAY, DELTA, float, bf16_t>(mode, p, shmem, s);
    if (st == BF16 && it == F32) return launch_combo<D, BV, DECAY, DELTA, bf16_t, float>(mode, p, shmem, s);
    if (st == BF16 && it == BF16) return launch_combo<D, BV, DECAY, DELTA, bf16_t, bf16_t>(mode, p, shmem, s);
    return hipErrorInvalidValue;
}

template <int D, int BV>
hipError_t launch_step_d(int mode, int decay, int update, int st, int it, const StepParams &p,
                         size_t shmem, hipStream_t s) {
    const bool delta = update != 0;
    switch (decay) {
    case DECAY_NONE:
        return delta ? launch_dtypes<D, BV, DECAY_NONE, true>(mode, st, it, p, shmem, s)
                     : launch_dtypes<D, BV, DECAY_NONE, false>(mode, st, it, p, shmem, s);
    case DECAY_SCALAR:
        return delta ? launch_dtypes<D, BV, DECAY_SCALAR, true>(mode, st, it, p, shmem, s)
                     : launch_dtypes<D, BV, DECAY_SCALAR, false>(mode, st, it, p, shmem, s);
    case DECAY_PER_KEY:
        return delta ? launch_dtypes<D, BV, DECAY_PER_KEY, true>(mode, st, it, p, shmem, s)
                     : launch_dtypes<D, BV, DECAY_PER_KEY, false>(mode, st, it, p, shmem, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dl
