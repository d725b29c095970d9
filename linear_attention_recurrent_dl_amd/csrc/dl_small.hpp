// Narrow-tile decode and eager kernels: value tiles of 16 or 32 columns (the
// library's default at small batch), scalar or no decay.
//
// Same arithmetic as dl_step_kernel ([DL] Eq. 3, the append-merge cycle and
// the GPU-execution section), laid out for launches whose blocks each have a
// CU to themselves.  There a wave issues about one instruction per four
// cycles and every barrier is a full stop, so the block is built around one
// barrier before the output:
//
//   - each thread takes q and k on its own tile rows straight from the token
//     arrays (the decayed q~ and k~ need no LDS round trip), so the tile's
//     projections start as soon as the tile lands;
//   - the log is replayed by entries: a lane holds two key chunks of one
//     entry (TPE2 lanes per entry) and that entry's value factor on UPL
//     columns of the tile; the entry's replay coefficients (DPP sums over its
//     lanes, weighted e^{l'-Lam_i}) multiply the value factor in the same
//     lanes, and the products are summed over the wave's entries with row
//     swaps, so no coefficient crosses a wave;
//   - the per-wave tile and log partial sums meet in LDS behind the one
//     barrier, where the output lanes finish the columns.
//
// The live length always comes from the device counter (a scalar load issued
// with the token loads; the host's value in the slot word is not needed), and
// the first round of log entries is loaded for the log's whole capacity while
// the counter is in flight.  Keys, value factors and weights reach LDS only
// for a merge, which needs them row by row.
#pragma once

namespace dl {

// UPL consecutive value-factor elements of type T, as fp32 (UPL * sizeof(T) in
// {2, 4, 8, 16, 32} bytes, aligned to the smaller of that and 16).
template <typename T, int UPL>
__device__ __forceinline__ void ld_cols(const T *src, float (&x)[UPL]) {
    constexpr int BYTES = UPL * (int)sizeof(T);
    if constexpr (sizeof(T) == 4) {
        if constexpr (UPL == 1) {
            x[0] = *reinterpret_cast<const float *>(src);
        } else if constexpr (UPL == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(src);
            x[0] = v.x;
            x[1] = v.y;
        } else {
            static_assert(UPL % 4 == 0 && UPL <= 8, "fp32 columns");
#pragma unroll
            for (int c = 0; c < UPL; c += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(src + c);
                x[c] = v.x;
                x[c + 1] = v.y;
                x[c + 2] = v.z;
                x[c + 3] = v.w;
            }
        }
    } else {
        constexpr int NWD = BYTES >= 4 ? BYTES / 4 : 1;
        uint32_t w[NWD];
        if constexpr (BYTES == 2) {
            w[0] = *reinterpret_cast<const uint16_t *>(src);
        } else if constexpr (BYTES == 4) {
            w[0] = *reinterpret_cast<const uint32_t *>(src);
        } else if constexpr (BYTES == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(src);
            w[0] = v.x;
            w[1] = v.y;
        } else {
            static_assert(BYTES % 16 == 0 && BYTES <= 32, "bf16 columns");
#pragma unroll
            for (int c = 0; c < BYTES / 16; ++c) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src + 8 * c);
                w[4 * c] = v.x;
                w[4 * c + 1] = v.y;
                w[4 * c + 2] = v.z;
                w[4 * c + 3] = v.w;
            }
        }
#pragma unroll
        for (int u = 0; u < UPL; ++u) x[u] = __uint_as_float((u & 1 ? w[u / 2] >> 16 : w[u / 2] & 0xFFFFu) << 16);
    }
}

// ---- reduce-scatter across the lanes of a wave.  R values per lane are
// summed over the lanes that differ only in the lane-index bits of MASK:
// bits 5 and 4 by the row swaps, bits 3, 1 and 0 by DPP (bit 2 has no DPP
// partner by exclusive-or).  A swap of two values hands each half of the
// wave the sum of one of them, so every swap level halves the values a lane
// holds for one swap and one add per pair; a DPP level does the same where
// the select it needs saves instructions over the levels left.  Lanes whose
// bit is 0 keep the sums of the even-numbered values, the others those of the
// odd-numbered.  All lanes of the wave must be active.

// instructions to sum r values over k DPP levels, halving where it pays
constexpr int rs_best(int r, int k) {
    if (k == 0) return 0;
    if (r == 1) return k;
    const int plain = r * k, split = 3 * (r / 2) + rs_best(r / 2, k - 1);
    return plain < split ? plain : split;
}
constexpr bool rs_split_dpp(int r, int k) {
    return r >= 2 && 3 * (r / 2) + rs_best(r / 2, k - 1) < r * k;
}
// DPP levels of MASK at bits <= bit
constexpr int rs_dpp_levels(int mask, int bit) {
    int k = 0;
    for (int b = bit < 3 ? bit : 3; b >= 0; --b) k += (mask >> b) & 1;
    return k;
}
// values per lane left after the levels of MASK, starting from r
constexpr int rs_left(int r, int mask) {
    for (int b = 5; b >= 0; --b) {
        if (!((mask >> b) & 1)) continue;
        if (b >= 4 ? r >= 2 : rs_split_dpp(r, rs_dpp_levels(mask, b))) r /= 2;
    }
    return r;
}

// x of lane ^ (1 << B) inside a row, B in {0, 1, 3}
template <int B>
__device__ __forceinline__ float from_lane_xor(float x) {
    static_assert(B == 0 || B == 1 || B == 3, "exclusive-or partner by DPP");
    if constexpr (B == 0) return dpp_f32<kDppQuadXor1>(x);
    else if constexpr (B == 1) return dpp_f32<kDppQuadXor2>(x);
    else return dpp_f32<kDppRowRor + 8>(x);
}

// Levels at bits BIT, BIT - 1, .., 0.  Returns the lane's offset: value m
// left in the lane is the sum of original value m * 2^S' + offset, S' the
// number of halving levels.
template <int N, int R, int MASK, int BIT, int S>
__device__ __forceinline__ int reduce_scatter(float (&x)[N], const int lane, const int sel) {
    static_assert(!((MASK >> 2) & 1), "no exclusive-or partner for lane bit 2");
    if constexpr (BIT < 0) {
        return sel;
    } else if constexpr (!((MASK >> BIT) & 1)) {
        return reduce_scatter<N, R, MASK, BIT - 1, S>(x, lane, sel);
    } else if constexpr (BIT >= 4) {
        if constexpr (R >= 2) {
#pragma unroll
            for (int m = 0; m < R / 2; ++m) {
                const uint32_t a = __float_as_uint(x[2 * m]), b = __float_as_uint(x[2 * m + 1]);
                if constexpr (BIT == 5) {
                    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
                    x[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                } else {
                    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
                    x[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                }
            }
            return reduce_scatter<N, R / 2, MASK, BIT - 1, S + 1>(x, lane, sel | (((lane >> BIT) & 1) << S));
        } else {
            x[0] = BIT == 5 ? sum_rows_xor2(x[0]) : sum_rows_xor1(x[0]);
            return reduce_scatter<N, R, MASK, BIT - 1, S>(x, lane, sel);
        }
    } else if constexpr (rs_split_dpp(R, rs_dpp_levels(MASK, BIT))) {
        const bool hi = (lane >> BIT) & 1;
#pragma unroll
        for (int m = 0; m < R / 2; ++m) {
            const float keep = hi ? x[2 * m + 1] : x[2 * m], send = hi ? x[2 * m] : x[2 * m + 1];
            x[m] = keep + from_lane_xor<BIT>(send);
        }
        return reduce_scatter<N, R / 2, MASK, BIT - 1, S + 1>(x, lane, sel | ((int)hi << S));
    } else {
#pragma unroll
        for (int m = 0; m < R; ++m) x[m] += from_lane_xor<BIT>(x[m]);
        return reduce_scatter<N, R, MASK, BIT - 1, S>(x, lane, sel);
    }
}

template <int D, int BV, int DECAY, bool DELTA, typename ST, typename IT, bool EAGER>
__global__ void __launch_bounds__((Tile<D, BV, ST>::NT))
dl_small_kernel(const int32_t H_v, const int32_t H_k, const int32_t C, const uint32_t gdiv, const StepParams p) {
    using G = Tile<D, BV, ST>;
    using BT = typename std::conditional<DELTA, float, IT>::type;   // value-factor storage
    constexpr int NT = G::NT, VEC = G::VEC, CG = G::CG, RG = G::RG, RPT = G::RPT, NW = G::NW;
    constexpr int NV = D / BV;
    constexpr int KV = 16 / (int)sizeof(IT);      // key elements per 16-byte chunk
    constexpr int CPE = D / KV;                   // key chunks per log entry
    constexpr int TPE2 = CPE / 2;                 // lanes per log entry (two chunks each)
    constexpr int EPR = NT / TPE2;                // log entries per round
    constexpr int UPL = BV / TPE2;                // value-factor columns per lane
    constexpr bool SCALAR = DECAY == DECAY_SCALAR;
    static_assert(DECAY != DECAY_PER_KEY, "scalar or no decay");
    static_assert(!G::RAGGED && RPT * RG == D, "tile rows");
    static_assert(UPL >= 1 && UPL * sizeof(BT) <= 32, "value-factor columns");
    static_assert(TPE2 >= 2 && TPE2 <= 64 && 64 % TPE2 == 0, "entry lanes within a wave");

    // partial projections per wave: [tile, log][wave][q, k][column], read
    // back as float4 slots, NQ = BV / 2 per (source, wave)
    constexpr int NQ = BV / 2;
    __shared__ __align__(16) float s_part[2][NW][2][BV];
    __shared__ __align__(16) float s_b[BV];             // b on the tile's columns (merge broadcast)
    __shared__ float s_w[kMaxLogCap + 1];               // e^{l'-Lam_i} (merge)
    extern __shared__ float4 s_dyn[];                   // merge: K [n][D] (IT), then U [n][BV] (BT)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // (unsigned index math with no branch: the argument fetch below then
    // shares a block with it, and the scheduler issues the fetch first)
    const uint32_t e = blockIdx.y;                      // batch entry of this launch
    const uint32_t sword = p.slots[e];
    const uint32_t ux = xcd_unit_u(blockIdx.x, (uint32_t)H_v * NV);
    const int h = (int)(ux / NV), vt = (int)(ux % NV);  // v-head, value tile
    const int eh = (int)e * H_v + h;
    const int c0 = vt * BV;                             // first column of the tile
    const int g = (int)qk_head((uint32_t)h, gdiv);
    const bool kwriter = first_of_group((uint32_t)h, gdiv);
    asm volatile("" ::"s"(p.base), "s"(p.klog), "s"(p.ulog), "s"(p.lamlog), "s"(p.nlog), "s"(p.q), "s"(p.k),
                 "s"(p.v), "s"(p.lam), "s"(p.beta), "s"(p.out), "s"(sword));
    const uint32_t slot = sword & kSlotMask;
    const uint32_t sh32 = slot * (uint32_t)H_v + (uint32_t)h;
    const uint32_t gk32 = slot * (uint32_t)H_k + (uint32_t)g;
    const uint32_t shv = sh32 * NV + (uint32_t)vt;      // (slot-head, value tile)
    const size_t shC = (size_t)sh32 * (uint32_t)C;      // the slot-head's first log entry
    const size_t gkC = (size_t)gk32 * (uint32_t)C;      // the q/k head's first key-log entry
    const uint32_t ek = (uint32_t)e * H_k + g;          // token row of q, k
    const uint32_t ev = (uint32_t)eh;                   // token row of v, lambda, beta, output
    // tile geometry: a thread holds one 16-byte chunk (VEC columns) of RPT
    // tile rows.  The column group sits in lane bits 2-3 (CG = 2: bit 2;
    // CG = 8: bits 1-3), the wave's 64 / CG row groups in the others, so that
    // the row sums reduce-scatter over lane bits 5, 4, 1 and 0 (row swaps and
    // quad DPP); a 16-lane row still covers whole tile rows of contiguous bytes
    static_assert(CG == 2 || CG == 4 || CG == 8, "column groups");
    constexpr int LPG = 64 / CG;                        // row groups per wave
    constexpr int CGB = CG == 8 ? 1 : 2;                // lowest lane bit of the column group
    constexpr int CGL = CG == 2 ? 1 : (CG == 4 ? 2 : 3);
    constexpr int TMASK = 0x3F & ~((CG - 1) << CGB);    // lane bits the row sums run over
    const int cg = (lane >> CGB) & (CG - 1);
    const int rg = wave * LPG + ((lane & ((1 << CGB) - 1)) | ((lane >> (CGB + CGL)) << CGB));
    const int jk = tid % TPE2;                          // the lane's place within its log entry
    const bool owner = vt == 0;                         // writes the tile-shared log metadata

    // output and appended value factor, one column per lane of wave 0.  The
    // partial sums are read back as float4 slots (a q/k row of BV / 4 slots,
    // C4B lane bits, then the q/k bit) and reduce-scattered over the lane bits
    // above, so that lane l ends with y~_q (q/k bit 0) or y~_k (bit 1) of
    // column 4 (l mod BV/4) + (lane bit 5) + 2 (lane bit 4).  Lanes whose other
    // bits (bit 3 at 16 columns) are 0 own their column.
    constexpr int C4B = BV == 16 ? 2 : 3;
    static_assert(BV == 4 << C4B, "16 or 32 columns");
    constexpr int SMASK = 0x3F & ~((2 << C4B) - 1);    // lane bits the slot sums run over
    const bool oq = !((lane >> C4B) & 1);               // holds y~_q: output lane, else value-factor lane
    const bool oown = (lane & SMASK & 0x0F) == 0;
    const int ocol = 4 * (lane & ((1 << C4B) - 1)) + ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1);

    // ---- loads, all issued before any is consumed (v of the lane's output
    // columns too: a load only the output lanes consume would be sunk behind
    // the others)
    // the counter and the per-head scalars go out first, through the scalar
    // path (their round trip then overlaps the vector loads' issue; the
    // scheduling barrier keeps the compiler from moving them behind)
    typedef const __attribute__((address_space(4))) int32_t *cint_p;
    typedef const __attribute__((address_space(4))) float *cfloat_p;
    // (the eager kernel, with no counter to wait for, measured faster with
    // vector loads of the scalars)
    int n_dev = 0;
    float lam = 0.f, beta = 0.f;
    if constexpr (!EAGER) {
        n_dev = ((cint_p)(size_t)p.nlog)[shv];
        if constexpr (SCALAR) lam = ((cfloat_p)(size_t)p.lam)[ev];
        if constexpr (DELTA) beta = ((cfloat_p)(size_t)p.beta)[ev];
        __builtin_amdgcn_sched_barrier(0);
    } else {
        if constexpr (SCALAR) lam = p.lam[ev];
        if constexpr (DELTA) beta = p.beta[ev];
    }
    const IT *qg = reinterpret_cast<const IT *>(p.q) + ek * D;
    const IT *kg = reinterpret_cast<const IT *>(p.k) + ek * D;
    float qr[RPT], kr[RPT];                             // q and a (= k) on the thread's tile rows
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        qr[j] = to_f32(qg[rg + RG * j]);
        kr[j] = to_f32(kg[rg + RG * j]);
    }
    const float vo = to_f32(reinterpret_cast<const IT *>(p.v)[ev * D + c0 + ocol]);   // v on the lane's column
    uint4 qc[2], ac[2];                                 // q and a on the lane's two key chunks
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        qc[c] = *reinterpret_cast<const uint4 *>(qg + (jk * 2 + c) * KV);
        ac[c] = *reinterpret_cast<const uint4 *>(kg + (jk * 2 + c) * KV);
    }
    const IT *klog = reinterpret_cast<const IT *>(p.klog);
    const BT *ulog = reinterpret_cast<const BT *>(p.ulog);
    const float *lamlog = p.lamlog;
    const uint4 *kb = reinterpret_cast<const uint4 *>(klog + gkC * D);
    const BT *ub = ulog + shC * D + c0;
    // round 0 of the log for the whole capacity (C >= 1 in a decode launch):
    // entry i0 = tid / TPE2 (clamped), its snapshot, its value factor on the
    // lane's columns; lane i of every wave also holds snapshot i
    float lam_w = 0.f, le0 = 0.f, uu0[UPL];
    uint4 kc0[2];
    if constexpr (!EAGER) {
        const int i0 = min(tid / TPE2, C - 1);
        if constexpr (SCALAR) {
            lam_w = lamlog[shC + min(lane, C - 1)];
            le0 = lamlog[shC + i0];
        }
        const uint4 *src = kb + (size_t)i0 * CPE + jk * 2;
        kc0[0] = src[0];
        kc0[1] = src[1];
        ld_cols<BT, UPL>(ub + (size_t)i0 * D + jk * UPL, uu0);
    }
    const ST *tbase = reinterpret_cast<const ST *>(p.base) + (size_t)shv * (D * BV);
    const uint32_t toff = (uint32_t)((rg * BV + cg * VEC) * sizeof(ST));
    constexpr uint32_t TROW = RG * BV * sizeof(ST);     // bytes between a thread's rows
    uint4 tile[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) tile[j] = ld16(tbase, toff + j * TROW);

    // ---- live length, l' = l_bar + lambda
    int n = 0;
    if constexpr (!EAGER) n = min(max(__builtin_amdgcn_readfirstlane(n_dev), 0), C);
    const bool merge = EAGER || n == C;
    float lbar = 0.f;
    if constexpr (SCALAR && !EAGER) {                   // newest snapshot, from lane n - 1 (uniform n)
        // (read unconditionally: a read inside a branch on n lets the compiler
        // sink the snapshot load behind every other load)
        const float lw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_w), max(n - 1, 0)));
        lbar = n > 0 ? lw : 0.f;
    }
    const float lp = lbar + lam;
    const float gg = SCALAR ? __expf(lp) : 1.f;         // e^{l'}

    // ---- log replay by entries (decode)
    char *s_log = reinterpret_cast<char *>(s_dyn);
    const IT *s_lk = reinterpret_cast<const IT *>(s_log);
    BT *s_lu = reinterpret_cast<BT *>(s_log + (size_t)C * CPE * 16);
    // a live entry's key chunks, value factors and weight into LDS (merge)
    auto stage_entry = [&](const int i, const uint4 (&kc)[2], const float (&uu)[UPL], const float w) {
        uint4 *dk = reinterpret_cast<uint4 *>(s_log) + (size_t)i * CPE + jk * 2;
        dk[0] = make_uint4(kc[0].x, kc[0].y, kc[0].z, kc[0].w);
        dk[1] = make_uint4(kc[1].x, kc[1].y, kc[1].z, kc[1].w);
#pragma unroll
        for (int u = 0; u < UPL; ++u) s_lu[i * BV + jk * UPL + u] = from_f32<BT>(uu[u]);
        if (jk == 0) s_w[i] = w;
    };
    float w0 = 1.f;                                     // weight of the lane's round-0 entry
    if constexpr (!EAGER) {
        float lq[UPL], lk[UPL];
#pragma unroll
        for (int u = 0; u < UPL; ++u) lq[u] = lk[u] = 0.f;
        // one round: every lane of the block, uniform r (DPP sums)
        // one round, returning the entry's weight: every lane of the block,
        // uniform r (DPP sums), no branch (so that the compiler can interleave
        // it with the tile's projections)
        auto replay_round = [&](const int r, const uint4 (&kc)[2], const float le, const float (&uu)[UPL]) -> float {
            const int i = r * EPR + tid / TPE2;
            float pq = dot16<IT>(kc[0], qc[0]) + dot16<IT>(kc[1], qc[1]);
            float pk = 0.f;
            if constexpr (DELTA) pk = dot16<IT>(kc[0], ac[0]) + dot16<IT>(kc[1], ac[1]);
            pq = group_sum<TPE2>(pq);
            if constexpr (DELTA) pk = group_sum<TPE2>(pk);
            // (computed in every lane, zero past the live log: a snapshot or
            // value factor used only under a branch would have its load sunk
            // behind all the others)
            // Entries past the live log may hold anything (memory never
            // written yet), so their products are selected away, not scaled by 0.
            const bool live = i < n;
            const float w = SCALAR ? __expf(lp - le) : 1.f;
            const float cq = pq * w, ck = pk * w;
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                const float tq = cq * uu[u];
                lq[u] += live ? tq : 0.f;
                if constexpr (DELTA) {
                    const float tk = ck * uu[u];
                    lk[u] += live ? tk : 0.f;
                }
            }
            return w;
        };
        w0 = replay_round(0, kc0, le0, uu0);
        for (int r = 1; r * EPR < n; ++r) {             // logs longer than one round
            const int i = r * EPR + tid / TPE2;
            uint4 kc[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
            float le = 0.f, uu[UPL];
#pragma unroll
            for (int u = 0; u < UPL; ++u) uu[u] = 0.f;
            if (i < n) {
                const uint4 *src = kb + (size_t)i * CPE + jk * 2;
                kc[0] = src[0];
                kc[1] = src[1];
                if constexpr (SCALAR) le = lamlog[shC + i];
                ld_cols<BT, UPL>(ub + (size_t)i * D + jk * UPL, uu);
            }
            const float w = replay_round(r, kc, le, uu);
            if (merge && i < n) stage_entry(i, kc, uu, w);
        }
        // sum over the wave's entries: lanes that agree modulo TPE2 hold the same columns
        if constexpr (TPE2 >= 8) {
            // reduce-scatter over lane bits log2(TPE2) .. 5; every lane stores what it holds
            constexpr int NR = DELTA ? 2 * UPL : UPL;
            constexpr int EMASK = 0x3F & ~(TPE2 - 1);
            float xs[NR];
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                xs[u] = lq[u];
                if constexpr (DELTA) xs[UPL + u] = lk[u];
            }
            const int sel = reduce_scatter<NR, NR, EMASK, 5, 0>(xs, lane, 0);
            constexpr int RL = rs_left(NR, EMASK);
#pragma unroll
            for (int m = 0; m < RL; ++m) {
                const int t = m * (NR / RL) + sel;
                s_part[1][wave][t / UPL][jk * UPL + t % UPL] = xs[m];
            }
        } else {
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                lq[u] = strided_sum<TPE2>(lq[u]);
                if constexpr (DELTA) lk[u] = strided_sum<TPE2>(lk[u]);
            }
            if (lane < TPE2) {
#pragma unroll
                for (int u = 0; u < UPL; ++u) {
                    s_part[1][wave][0][jk * UPL + u] = lq[u];
                    s_part[1][wave][1][jk * UPL + u] = lk[u];
                }
            }
        }
    }

    // ---- tile projections: y~ = S_bar^T q~, S_bar^T k~ over the thread's rows
    float accq[VEC], acck[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) accq[c] = acck[c] = 0.f;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        float x[VEC];
        unpack_f32<ST, VEC>(tile[j], x);
        const float qd = gg * qr[j], kd = gg * kr[j];
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            accq[c] += x[c] * qd;
            if constexpr (DELTA) acck[c] += x[c] * kd;
        }
    }
    {
        // row sums of y~_q (and y~_k) on the thread's VEC columns, scattered
        // over the lanes of the column group; every lane stores what it holds
        // (lanes holding the same sum store the same value)
        constexpr int NV = DELTA ? 2 * VEC : VEC;
        float xs[NV];
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            xs[c] = accq[c];
            if constexpr (DELTA) xs[VEC + c] = acck[c];
        }
        const int sel = reduce_scatter<NV, NV, TMASK, 5, 0>(xs, lane, 0);
        constexpr int RL = rs_left(NV, TMASK);
#pragma unroll
        for (int m = 0; m < RL; ++m) {
            const int t = m * (NV / RL) + sel;          // value index: t / VEC = q or k, t % VEC = column
            s_part[0][wave][t / VEC][cg * VEC + t % VEC] = xs[m];
        }
    }
    // a . q, from the first entry's lanes, in lanes 0-15 (the column lanes)
    float aq = 0.f;
    if (tid < TPE2) aq = dot16<IT>(qc[0], ac[0]) + dot16<IT>(qc[1], ac[1]);
    aq = group_sum<16>(aq);
    // stores that need no reduced value: the appended key (first v-head of
    // the q/k group, first tile) and decay snapshot, the live-length counter
    if constexpr (!EAGER) {
        if (!merge && owner) {
            if (kwriter && tid < TPE2) {
                uint4 *dk = reinterpret_cast<uint4 *>(reinterpret_cast<IT *>(p.klog) + (gkC + n) * D) + jk * 2;
                dk[0] = ac[0];
                dk[1] = ac[1];
            }
            if constexpr (SCALAR) {
                if (tid == 0) p.lamlog[shC + n] = lp;
            }
        }
        if (tid == 0) p.nlog[shv] = merge ? 0 : n + 1;
    }
    __syncthreads();

    // ---- output and appended value factor (wave 0), one column per lane
    if (wave != 0) {
        if (!merge) return;
    } else {
    constexpr int NSL = 2 * NW * NQ;                   // slots
    constexpr int SPL = (NSL + 63) / 64;               // slots per lane
    static_assert(64 % NQ == 0 && NQ == 2 << C4B, "partial-sum slots");
    static_assert(rs_left(4, SMASK) == 1, "one column per lane");
    const float4 *slots = reinterpret_cast<const float4 *>(&s_part[0][0][0][0]);
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
        const int idx = lane + 64 * s;
        if (idx < (EAGER ? NW * NQ : NSL)) {            // (eager: no log half)
            const float4 a = slots[idx];
            r[0] += a.x; r[1] += a.y; r[2] += a.z; r[3] += a.w;
        }
    }
    // sources and waves summed, the four columns scattered over lane bits 5, 4
    reduce_scatter<4, 4, SMASK, 5, 0>(r, lane, 0);
    const float y = r[0];
    // y~_k of an output lane's column sits BV/4 lanes up, in the same row
    // (moved while every lane of the wave is active: DPP reads no lane that
    // EXEC disables); a . q from lane 0
    const float yup = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0x100 + BV / 4, 0xf, 0xf, false));
    const float aqs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(aq), 0));
    const float b = DELTA ? beta * (vo - (oq ? yup : y)) : vo;
    if (oown) {
        if (oq) {
            if (merge) s_b[ocol] = b;
            __builtin_nontemporal_store(y + aqs * b, reinterpret_cast<float *>(p.out) + (size_t)ev * D + c0 + ocol);
        } else if (!EAGER && !merge) {
            // (a cached store: the next steps read the entry back, and a
            // streaming store measured 0.6% slower at batch 1)
            reinterpret_cast<BT *>(p.ulog)[(shC + n) * D + c0 + ocol] = from_f32<BT>(b);
        }
    }
    if (!merge) return;
    }

    // ---- merge (eager: every step): S_bar <- e^{l'} S_bar + sum_i (e^{l'-Lam_i} K_i) U_i^T + a b^T,
    // from the tile still in registers; the first round of live entries is
    // staged here, from registers (later rounds were staged as they came)
    if constexpr (!EAGER) {
        if (tid / TPE2 < n) stage_entry(tid / TPE2, kc0, uu0, w0);
    }
    __syncthreads();
    float bcol[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) bcol[c] = s_b[cg * VEC + c];
    float acc[RPT][VEC];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        unpack_f32<ST, VEC>(tile[j], acc[j]);
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[j][c] = gg * acc[j][c] + kr[j] * bcol[c];
    }
    if constexpr (!EAGER) {
        for (int i = 0; i < n; ++i) {
            float u[VEC];
            lds_f32<BT, VEC>(s_lu + i * BV + cg * VEC, u);
            const float w = s_w[i];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const float kt = to_f32(s_lk[i * D + rg + RG * j]) * w;
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[j][c] += kt * u[c];
            }
        }
    }
    ST *basew = const_cast<ST *>(tbase);
#pragma unroll
    for (int j = 0; j < RPT; ++j) st16(basew, toff + j * TROW, pack_16<ST, VEC>(acc[j]));
}

}  // namespace dl
