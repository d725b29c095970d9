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
//   2. token inputs go to LDS kWindowChunk steps at a time (double buffered;
//      the next chunk's loads are in flight during the current one, and a . q
//      and e^{lambda} are formed once per step at staging); then per step,
//      with one barrier:
//        P = D(lambda_w) S on the thread's rows; y_q = P^T q, y_k = P^T k by
//        per-thread FMAs, DPP / row-swap sums across the row groups of a wave
//        and an LDS sum across waves (double buffered by step parity); every
//        thread forms b on its own columns (delta: b = beta (v - y_k); plain:
//        the given b), updates S <- P + a b^T, and the first row group writes
//        o = y_q + (a . q) b
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
    constexpr int KC = kWindowChunk;
    static_assert(VEC % 4 == 0, "columns per thread in float4 groups");
    static_assert(KC >= 2, "a chunk is restaged after its buffer's last reader has passed a barrier");

    __shared__ __align__(16) float s_red[2][NW][2][BV];   // cross-wave partials, by step parity
    __shared__ float s_lam[kMaxLogCap + 1];         // scalar snapshots
    // dynamic: the live log as stored (step 1), then the token buffers (step 2)
    extern __shared__ float4 s_dyn[];

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
    // token buffer layout (floats): q [KC][D], a [KC][D], e^{lambda} [KC][D]
    // (per key), v [KC][BV], e^{lambda} [KC] (scalar), beta [KC], a . q [KC]
    constexpr int OQ = 0, OK = KC * D, OG = 2 * KC * D, OV = OG + (PERKEY ? KC * D : 0);
    constexpr int OGS = OV + KC * BV, OB = OGS + KC, OKQ = OB + KC;
    constexpr int TB = OKQ + 2 * KC;                    // = window_token_floats
    constexpr int MQ = (KC * D + NT - 1) / NT;          // q / a / lambda elements per thread and chunk
    constexpr int MV = (KC * BV + NT - 1) / NT;         // v elements per thread and chunk
    float *tok = reinterpret_cast<float *>(s_dyn);
    float rq[MQ], rk[MQ], rl[MQ], rv[MV], rs = 0.f, rb = 0.f;
#pragma unroll
    for (int m = 0; m < MQ; ++m) rq[m] = rk[m] = rl[m] = 0.f;
#pragma unroll
    for (int m = 0; m < MV; ++m) rv[m] = 0.f;
    const int W = p.W;
    auto load_chunk = [&](int w0) {                     // steps w0 .. w0 + KC - 1 into registers
        const int cnt = min(KC, W - w0);
#pragma unroll
        for (int m = 0; m < MQ; ++m) {
            const int x = tid + m * NT, j = x / D, r = x - j * D;
            if (x < KC * D && j < cnt) {
                const size_t ew = (size_t)(w0 + j) * sB + e;
                const size_t qo = (ew * p.H_k + g) * D + r;
                rq[m] = to_f32(reinterpret_cast<const IT *>(p.q)[qo]);
                rk[m] = to_f32(reinterpret_cast<const IT *>(p.k)[qo]);
                if constexpr (PERKEY) rl[m] = p.lam[(ew * H_v + h) * D + r];
            }
        }
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const int x = tid + m * NT, j = x / BV, c = x - j * BV;
            if (x < KC * BV && j < cnt)
                rv[m] = to_f32(reinterpret_cast<const IT *>(p.v)[(((size_t)(w0 + j) * sB + e) * H_v + h) * D + c0 + c]);
        }
        if (tid < cnt) {
            const size_t ew = (size_t)(w0 + tid) * sB + e;
            if constexpr (SCALAR) rs = p.lam[ew * H_v + h];
            if constexpr (DELTA) rb = p.beta[ew * H_v + h];
        }
    };
    auto store_chunk = [&](float *T) {
#pragma unroll
        for (int m = 0; m < MQ; ++m) {
            const int x = tid + m * NT;
            if (x < KC * D) {
                T[OQ + x] = rq[m];
                T[OK + x] = rk[m];
                if constexpr (PERKEY) T[OG + x] = __expf(rl[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const int x = tid + m * NT;
            if (x < KC * BV) T[OV + x] = rv[m];
        }
        if (tid < KC) {
            T[OGS + tid] = SCALAR ? __expf(rs) : 1.f;
            T[OB + tid] = rb;
        }
    };
    load_chunk(0);
    __syncthreads();                                    // the log is consumed: its LDS takes the tokens
    store_chunk(tok);
    __syncthreads();
    int buf = 0;
    for (int w0 = 0; w0 < W; w0 += KC) {
        const int cnt = min(KC, W - w0);
        const bool more = w0 + KC < W;
        if (more) load_chunk(w0 + KC);                  // in flight during this chunk
        float *T = tok + buf * TB;
        // a . q of the chunk's steps, wave by wave; read after the steps' barriers
        for (int j = wave; j < cnt; j += NW) {
            float pq = 0.f;
            for (int r = lane; r < D; r += 64) pq += T[OQ + j * D + r] * T[OK + j * D + r];
            pq = group_sum<64>(pq);
            if (lane == 0) T[OKQ + j] = pq;
        }
        for (int j = 0; j < cnt; ++j) {
            const int par = (w0 + j) & 1;
            const float *tq = T + OQ + j * D, *tk = T + OK + j * D, *tg = T + OG + j * D;
            const float gs = T[OGS + j];

            // P = D(lambda) S on this thread's rows; partial y_q = P^T q, y_k = P^T k
            float yq[VEC], yk[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) yq[c] = yk[c] = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rg + RG * i;
                if (!G::RAGGED || r < D) {
                    const float gr = PERKEY ? tg[r] : gs;
                    const float qr = tq[r], kr = tk[r];
#pragma unroll
                    for (int c = 0; c < VEC; ++c) {
                        acc[i][c] *= gr;
                        yq[c] += acc[i][c] * qr;
                        if constexpr (DELTA) yk[c] += acc[i][c] * kr;
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                yq[c] = strided_sum<CG>(yq[c]);
                if constexpr (DELTA) yk[c] = strided_sum<CG>(yk[c]);
            }
            if (lane < CG) {
#pragma unroll
                for (int c = 0; c < VEC; c += 4) {
                    *reinterpret_cast<float4 *>(&s_red[par][wave][0][cg * VEC + c]) =
                        make_float4(yq[c], yq[c + 1], yq[c + 2], yq[c + 3]);
                    if constexpr (DELTA)
                        *reinterpret_cast<float4 *>(&s_red[par][wave][1][cg * VEC + c]) =
                            make_float4(yk[c], yk[c + 1], yk[c + 2], yk[c + 3]);
                }
            }
            if (more && j == cnt - 1) store_chunk(tok + (buf ^ 1) * TB);   // the next chunk
            __syncthreads();

            // b on this thread's columns, S <- P + a b^T, o = y_q + (a . q) b
            const float beta = T[OB + j];
            float bcol[VEC];
#pragma unroll
            for (int c = 0; c < VEC; c += 4) {
                const float4 v4 = *reinterpret_cast<const float4 *>(T + OV + j * BV + cg * VEC + c);
                if constexpr (DELTA) {
                    float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int w2 = 0; w2 < NW; ++w2) {
                        const float4 a = *reinterpret_cast<const float4 *>(&s_red[par][w2][1][cg * VEC + c]);
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
            for (int i = 0; i < RPT; ++i) {
                const int r = rg + RG * i;
                if (!G::RAGGED || r < D) {
                    const float kr = tk[r];
#pragma unroll
                    for (int c = 0; c < VEC; ++c) acc[i][c] += kr * bcol[c];
                }
            }
            if (rg == 0) {
                const float aq = T[OKQ + j];
                float *dst = p.out + (((size_t)(w0 + j) * sB + e) * H_v + h) * D + c0 + cg * VEC;
#pragma unroll
                for (int c = 0; c < VEC; c += 4) {
                    float4 Y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int w2 = 0; w2 < NW; ++w2) {
                        const float4 a = *reinterpret_cast<const float4 *>(&s_red[par][w2][0][cg * VEC + c]);
                        Y.x += a.x; Y.y += a.y; Y.z += a.z; Y.w += a.w;
                    }
                    st16_stream(dst + c, 0,
                                make_uint4(__float_as_uint(Y.x + aq * bcol[c]), __float_as_uint(Y.y + aq * bcol[c + 1]),
                                           __float_as_uint(Y.z + aq * bcol[c + 2]),
                                           __float_as_uint(Y.w + aq * bcol[c + 3])));
                }
            }
        }
        buf ^= 1;
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
