// Resident-state window kernel for CDNA4 (gfx950): W consecutive decode steps
// of the same slots in one launch, each block's d_k x B_V tile of the state
// held in registers from the first step to the last.
//
// Sources: [DL] Eq. 3 (the per-step recurrence and output) and the
// logical-state equation (base plus decayed log); [FPGA] the persistent-state
// design, which keeps the whole state on chip while per-token inputs stream
// in.  On this GPU the registers of the blocks of one launch hold the state
// (2 MiB for 32 v-heads at d = 128 fills 128 blocks of 16 KiB); the token
// inputs of all W steps are in device memory before the launch, so the window
// applies where they are known together (a streamed token sequence, a run of
// draft tokens), not to one-token-at-a-time decoding driven by the model.
//
// Per block:
//   1. load the base tile and stage the live log in LDS; materialize the
//      logical state S = D(l_bar) S_bar + sum_i D(l_bar - Lam_i) K_i U_i^T in
//      registers (fp32)
//   2. for each step w (its token staged in LDS, double buffered, the next
//      step's inputs in flight):
//        P = D(lambda_w) S on the thread's rows; y_q = P^T q, y_k = P^T k by
//        per-thread FMAs, DPP / row-swap sums across the row groups of a wave
//        and an LDS sum across waves; every thread forms b on its own columns
//        (delta: b = beta (v - y_k); plain: the given b), updates
//        S <- P + a b^T and the first row group writes o = y_q + (a . q) b
//   3. write the tile back to the base and empty the log (n <- 0)
#pragma once

#include "dl_kernels.hpp"

namespace dl {

template <int D, int BV, int DECAY, bool DELTA, typename ST, typename IT>
__global__ void __launch_bounds__((Tile<D, BV, ST>::NT))
dl_window_kernel(const WindowParams p) {
    using G = Tile<D, BV, ST>;
    using BT = typename std::conditional<DELTA, float, IT>::type;   // value-factor storage
    constexpr int NT = G::NT, VEC = G::VEC, CG = G::CG, RG = G::RG, RPT = G::RPT, NW = G::NW;
    constexpr int NV = D / BV;
    constexpr int KV = 16 / (int)sizeof(IT);
    constexpr int UV = 16 / (int)sizeof(BT);
    constexpr int UCH = BV / UV;
    constexpr bool PERKEY = DECAY == DECAY_PER_KEY;
    constexpr bool SCALAR = DECAY == DECAY_SCALAR;
    static_assert(VEC % 4 == 0, "columns per thread in float4 groups");

    __shared__ float s_q[2][D];                     // q of the step (double buffered)
    __shared__ float s_k[2][D];                     // a (= k) of the step
    __shared__ float s_g[PERKEY ? 2 : 1][D];        // e^{lambda} per key
    __shared__ __align__(16) float s_v[2][BV];      // v (or the given b) on this tile's columns
    __shared__ __align__(16) float s_red[NW][2][BV];
    __shared__ float s_lam[kMaxLogCap + 1];         // scalar snapshots
    extern __shared__ float4 s_dyn[];               // the live log as stored

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    const int H_v = p.H_v, C = p.C;
    const size_t sB = (size_t)p.B;
    const int eh = unit / NV, vt = unit - eh * NV;      // (entry, v-head), value tile
    const int e = eh / H_v, h = eh - e * H_v;
    const int c0 = vt * BV;
    const int g = h / (H_v / p.H_k);
    const int slot = (int)(p.slots[e] & kSlotMask);
    const size_t sh = (size_t)slot * H_v + h;
    const size_t gk = (size_t)slot * p.H_k + g;
    const int cg = tid % CG, rg = tid / CG;

    // ---- 1. base tile, live log, logical state
    const ST *tbase = reinterpret_cast<const ST *>(p.base) + (sh * NV + vt) * (size_t)(D * BV);
    const uint32_t toff = (uint32_t)((rg * BV + cg * VEC) * sizeof(ST));
    constexpr uint32_t TROW = RG * BV * sizeof(ST);
    uint4 tile[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        if (!G::RAGGED || rg + RG * j < D) tile[j] = ld16(tbase, toff + j * TROW);
        else tile[j] = make_uint4(0, 0, 0, 0);
    }
    const int n = min(max(p.nlog[sh * NV + vt], 0), C);
    // chunk x of the log at byte 16 x: key factors [n][D], value factors on
    // this tile [n][BV], per-key snapshots [n][D]
    const int cK = n * D / KV, cU = n * UCH, cL = PERKEY ? n * D / 4 : 0;
    const int ctot = cK + cU + cL;
    char *s_log = reinterpret_cast<char *>(s_dyn);
    const IT *s_lk = reinterpret_cast<const IT *>(s_log);
    const BT *s_lu = reinterpret_cast<const BT *>(s_log + (size_t)cK * 16);
    const float *s_ll = reinterpret_cast<const float *>(s_log + (size_t)(cK + cU) * 16);
    if (n > 0) {
        const uint4 *kb = reinterpret_cast<const uint4 *>(reinterpret_cast<const IT *>(p.klog) + gk * C * D);
        const BT *ub = reinterpret_cast<const BT *>(p.ulog) + sh * C * D + c0;
        const uint4 *lb = reinterpret_cast<const uint4 *>(p.lamlog + sh * C * D);
        for (int x = tid; x < ctot; x += NT) {
            const uint4 *src;
            if (x < cK) {
                src = kb + x;
            } else if (x < cK + cU) {
                const int u = x - cK, i = u / UCH;
                src = reinterpret_cast<const uint4 *>(ub + (size_t)i * D + (u - i * UCH) * UV);
            } else {
                src = lb + (x - cK - cU);
            }
            const uint4 w = *src;
            *reinterpret_cast<uint4 *>(s_log + (size_t)x * 16) = make_uint4(w.x, w.y, w.z, w.w);
        }
        if constexpr (SCALAR) {
            if (tid < n) s_lam[tid] = p.lamlog[sh * C + tid];
        }
    }
    __syncthreads();

    float acc[RPT][VEC];
    const float lbs = (SCALAR && n > 0) ? s_lam[n - 1] : 0.f;   // scalar l_bar (newest snapshot)
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = rg + RG * j;
        const int rr = r < D ? r : 0;
        unpack_f32<ST, VEC>(tile[j], acc[j]);
        float gb = 1.f;
        if constexpr (SCALAR) gb = __expf(lbs);
        if constexpr (PERKEY) gb = n > 0 ? __expf(s_ll[(n - 1) * D + rr]) : 1.f;
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[j][c] *= gb;
    }
    for (int i = 0; i < n; ++i) {
        float u[VEC];
        lds_f32<BT, VEC>(s_lu + i * BV + cg * VEC, u);
        const float ws = SCALAR ? __expf(lbs - s_lam[i]) : 1.f;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg + RG * j;
            const int rr = r < D ? r : 0;
            float kt = to_f32(s_lk[i * D + rr]);
            if constexpr (PERKEY) kt *= __expf(s_ll[(n - 1) * D + rr] - s_ll[i * D + rr]);
            else kt *= ws;
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[j][c] += kt * u[c];
        }
    }

    // ---- 2. the steps
    float qv = 0.f, kv = 0.f, vv = 0.f, lv = 0.f, ls = 0.f, bs = 0.f;
    auto load_token = [&](int w) {
        const size_t ew = (size_t)w * sB + e;           // entry e of step w
        if (tid < D) {
            const size_t qo = (ew * p.H_k + g) * D + tid;
            qv = to_f32(reinterpret_cast<const IT *>(p.q)[qo]);
            kv = to_f32(reinterpret_cast<const IT *>(p.k)[qo]);
            if constexpr (PERKEY) lv = p.lam[(ew * H_v + h) * D + tid];
            if (tid < BV) vv = to_f32(reinterpret_cast<const IT *>(p.v)[(ew * H_v + h) * D + c0 + tid]);
        }
        if constexpr (SCALAR) ls = p.lam[ew * H_v + h];
        if constexpr (DELTA) bs = p.beta[ew * H_v + h];
    };
    load_token(0);
    for (int w = 0; w < p.W; ++w) {
        const int buf = w & 1;
        if (tid < D) {
            s_q[buf][tid] = qv;
            s_k[buf][tid] = kv;
            if constexpr (PERKEY) s_g[buf][tid] = __expf(lv);
            if (tid < BV) s_v[buf][tid] = vv;
        }
        const float gs = SCALAR ? __expf(ls) : 1.f;
        const float beta = bs;
        if (w + 1 < p.W) load_token(w + 1);
        __syncthreads();

        // P = D(lambda) S on this thread's rows; partial y_q = P^T q, y_k = P^T k
        float yq[VEC], yk[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) yq[c] = yk[c] = 0.f;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg + RG * j;
            if (!G::RAGGED || r < D) {
                const float gr = PERKEY ? s_g[PERKEY ? buf : 0][r] : gs;
                const float qr = s_q[buf][r], kr = s_k[buf][r];
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    acc[j][c] *= gr;
                    yq[c] += acc[j][c] * qr;
                    if constexpr (DELTA) yk[c] += acc[j][c] * kr;
                }
            }
        }
        // a . q, summed by every wave for itself
        float pq = 0.f;
        for (int r = lane; r < D; r += 64) pq += s_q[buf][r] * s_k[buf][r];
        const float aq = group_sum<64>(pq);
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            yq[c] = strided_sum<CG>(yq[c]);
            if constexpr (DELTA) yk[c] = strided_sum<CG>(yk[c]);
        }
        if (lane < CG) {
#pragma unroll
            for (int c = 0; c < VEC; c += 4) {
                *reinterpret_cast<float4 *>(&s_red[wave][0][cg * VEC + c]) =
                    make_float4(yq[c], yq[c + 1], yq[c + 2], yq[c + 3]);
                if constexpr (DELTA)
                    *reinterpret_cast<float4 *>(&s_red[wave][1][cg * VEC + c]) =
                        make_float4(yk[c], yk[c + 1], yk[c + 2], yk[c + 3]);
            }
        }
        __syncthreads();

        // b on this thread's columns, S <- P + a b^T, o = y_q + (a . q) b
        float bcol[VEC];
#pragma unroll
        for (int c = 0; c < VEC; c += 4) {
            const float4 v4 = *reinterpret_cast<const float4 *>(&s_v[buf][cg * VEC + c]);
            float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (DELTA) {
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) {
                    const float4 a = *reinterpret_cast<const float4 *>(&s_red[w2][1][cg * VEC + c]);
                    Y.x += a.x; Y.y += a.y; Y.z += a.z; Y.w += a.w;
                }
                bcol[c] = beta * (v4.x - Y.x);
                bcol[c + 1] = beta * (v4.y - Y.y);
                bcol[c + 2] = beta * (v4.z - Y.z);
                bcol[c + 3] = beta * (v4.w - Y.w);
            } else {
                bcol[c] = v4.x;
                bcol[c + 1] = v4.y;
                bcol[c + 2] = v4.z;
                bcol[c + 3] = v4.w;
            }
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg + RG * j;
            if (!G::RAGGED || r < D) {
                const float kr = s_k[buf][r];
#pragma unroll
                for (int c = 0; c < VEC; ++c) acc[j][c] += kr * bcol[c];
            }
        }
        if (rg == 0) {
            float *dst = p.out + (((size_t)w * sB + e) * H_v + h) * D + c0 + cg * VEC;
#pragma unroll
            for (int c = 0; c < VEC; c += 4) {
                float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) {
                    const float4 a = *reinterpret_cast<const float4 *>(&s_red[w2][0][cg * VEC + c]);
                    Y.x += a.x; Y.y += a.y; Y.z += a.z; Y.w += a.w;
                }
                st16_stream(dst + c, 0,
                            make_uint4(__float_as_uint(Y.x + aq * bcol[c]), __float_as_uint(Y.y + aq * bcol[c + 1]),
                                       __float_as_uint(Y.z + aq * bcol[c + 2]),
                                       __float_as_uint(Y.w + aq * bcol[c + 3])));
            }
        }
    }

    // ---- 3. the state back to the base; the log is empty
    ST *basew = const_cast<ST *>(tbase);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        if (!G::RAGGED || rg + RG * j < D) st16(basew, toff + j * TROW, pack_16<ST, VEC>(acc[j]));
    }
    if (tid == 0) p.nlog[sh * NV + vt] = 0;
}

template <int D, int BV, int DECAY, bool DELTA>
static hipError_t launch_window_dtypes(int st, int it, const WindowParams &p, size_t shmem, hipStream_t s) {
    constexpr int NT_F = Tile<D, BV, float>::NT, NT_B = Tile<D, BV, bf16_t>::NT;
    const dim3 grid(p.nunits);
    if (st == F32 && it == F32)
        dl_window_kernel<D, BV, DECAY, DELTA, float, float><<<grid, dim3(NT_F), shmem, s>>>(p);
    else if (st == F32 && it == BF16)
        dl_window_kernel<D, BV, DECAY, DELTA, float, bf16_t><<<grid, dim3(NT_F), shmem, s>>>(p);
    else if (st == BF16 && it == F32)
        dl_window_kernel<D, BV, DECAY, DELTA, bf16_t, float><<<grid, dim3(NT_B), shmem, s>>>(p);
    else if (st == BF16 && it == BF16)
        dl_window_kernel<D, BV, DECAY, DELTA, bf16_t, bf16_t><<<grid, dim3(NT_B), shmem, s>>>(p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D, int BV>
hipError_t launch_window_d(int decay, int update, int st, int it, const WindowParams &p, size_t shmem,
                           hipStream_t s) {
    const bool delta = update != 0;
    switch (decay) {
    case DECAY_NONE:
        return delta ? launch_window_dtypes<D, BV, DECAY_NONE, true>(st, it, p, shmem, s)
                     : launch_window_dtypes<D, BV, DECAY_NONE, false>(st, it, p, shmem, s);
    case DECAY_SCALAR:
        return delta ? launch_window_dtypes<D, BV, DECAY_SCALAR, true>(st, it, p, shmem, s)
                     : launch_window_dtypes<D, BV, DECAY_SCALAR, false>(st, it, p, shmem, s);
    case DECAY_PER_KEY:
        return delta ? launch_window_dtypes<D, BV, DECAY_PER_KEY, true>(st, it, p, shmem, s)
                     : launch_window_dtypes<D, BV, DECAY_PER_KEY, false>(st, it, p, shmem, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dl
