// gdn_prefill.h -- blockwise (chunked) prefill of the gated delta rule on gfx950.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates three
// distinct workload shapes": the recurrence can be evaluated by regrouping the updates
// into blocks that expose matrix operations and token-level parallelism.  For a chunk
// of n tokens that starts from state S0 (dv x dk), with gamma_r the running sum of the
// log-gates inside the chunk and Gamma_r = exp(gamma_r):
//
//   A[r,s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s),  s < r      (decay-masked Gram)
//   R      = (I + A)^-1                                           (unit lower triangular)
//   W      = R diag(beta Gamma) K,      Ut = R diag(beta) V         (state independent)
//   P[r,s] = exp(gamma_r - gamma_s) (q_r . k_s),  s <= r
//   U      = Ut - W S0^T                                          (deltas of the chunk)
//   O      = diag(Gamma) Q S0^T + P U
//   S_next = Gamma_{n-1} S0 + U^T diag(exp(gamma_{n-1} - gamma)) K
//
// Only exponentials of gamma_r - gamma_s with s <= r appear, so no factor can overflow.
//
// Kernel 1 (intra_chunk_kernel), one workgroup per (batch, key head, chunk), fully
// parallel.  The two Gram blocks K K^T and K Q^T are formed once on MFMA and kept in
// registers; then for each value head reading this key head: masks with that head's
// gates, (I + A) inverted in fp32 (16x16 diagonal blocks by substitution, then block
// back-substitution), W and Ut on MFMA.  Everything the scan needs goes to the workspace
// already arranged as MFMA operand fragments (see "Workspace layout").
//
// Kernel 2 (inter_chunk_kernel), one workgroup per (batch, value head, 16 state rows):
// rows of S evolve independently (each needs only its own entries of v), so a head's
// state is split into 16-row slices that never talk to each other.  The fp32 slice lives
// in MFMA accumulator registers for the whole scan and is written back once at the end
// ("Keep the recurrent state on chip": load the state once, carry it through the scan,
// write it after).  Each chunk's operands are fetched two chunks ahead into registers, so
// the chunk-to-chunk chain waits only on LDS exchanges and matrix-core latency.
//
// Workspace layout (E = element type; every fragment is 64 lanes x KPL elements, lane l
// holding row l % 16 and k-values (l / 16) * KPL + [0, KPL) of a 16 x KB tile):
//   W   [B][Hv][N][C/16][DK/KB] fragments   A operand of W S^T   (rows tokens, k = dk)
//   P   [B][Hv][N][C/16][NKC]   fragments   A operand of P U     (rows tokens, k = tokens)
//   KT  [B][Hk][N][DK/16][NKC]  fragments   A operand of K^T U'  (rows dk,     k = tokens)
//   Ut  [B][Hv][N][DV/16][C/16] accumulator tiles (lane: col l % 16, rows 4 (l/16) + [0,4))
//   gam [B][Hv][N][2][C] fp32 gate factors per chunk: exp(gamma_r), then exp(gamma_last - gamma_r)
//       (rows past the end repeat the last row's gamma)
// NKC = ceil(C / KB); k-values past the chunk are stored as zeros.
#pragma once

#include <type_traits>

#include "gdn_device.h"

namespace gdn {

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* state_in;
    void* o;
    float* state_out;
    void* W;
    void* Ut;
    void* P;
    void* KT;
    float* gam;   // gate factors (see the workspace layout)
    int B, T, Hk, Hv, N;  // N = number of chunks
};

constexpr int kThreads = 256;

template <typename E, int DK, int DV, int C>
struct PrefillShape {
    using X = Elem<E>;
    static constexpr int KB = X::KB, KPL = X::KPL;
    static constexpr int NT = C / 16;                       // token tiles per chunk
    static constexpr int NKD = DK / KB;                     // k-blocks over dk
    static constexpr int NKC = (C + KB - 1) / KB;           // k-blocks over a chunk's tokens
    static constexpr int FRAG = 64 * KPL;                   // elements per fragment
    static constexpr size_t W_PER_CHUNK = (size_t)NT * NKD * FRAG;
    static constexpr size_t P_PER_CHUNK = (size_t)NT * NKC * FRAG;
    static constexpr size_t KT_PER_CHUNK = (size_t)(DK / 16) * NKC * FRAG;
    static constexpr size_t UT_PER_CHUNK = (size_t)(DV / 16) * NT * 256;
};

// Index (tm, tn), tn <= tm, of the tt-th 16x16 tile of a lower-triangular tile grid.
__device__ __forceinline__ void lower_tile(int tt, int& tm, int& tn) {
    tm = 0;
    while (tt > tm) { tt -= tm + 1; ++tm; }
    tn = tt;
}

template <typename E>
__device__ __forceinline__ void store_frag(E* dst, const E* src) {
    if (Elem<E>::KPL == 8) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    else dst[0] = src[0];
}

template <typename E>
__device__ __forceinline__ void store4(E* dst, const E* v) {
    if (sizeof(E) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(v);
    else *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v);
}

// ------------------------------------------------------------------------------------
// Kernel 1: per-chunk, state-independent blocks.
// ------------------------------------------------------------------------------------
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename E, int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void intra_chunk_kernel(PrefillParams p) {
    using S = PrefillShape<E, DK, DV, C>;
    using X = Elem<E>;
    constexpr int KB = S::KB, KPL = S::KPL, NT = S::NT, NKD = S::NKD, NKC = S::NKC;
    constexpr int EPV = 16 / (int)sizeof(E);   // elements per 16-byte vector
    constexpr int LDK = DK + EPV;              // row pitch of K rows (elements)
    constexpr int LDV = DV + EPV;              // row pitch of V rows
    constexpr int CP = NKC * KB;               // chunk width padded to whole k-blocks
    constexpr int LDT = CP + EPV;              // row pitch of token-contiguous (transposed) tiles
    constexpr int LDA = C + 1;                 // fp32 A
    constexpr int LDR = CP + 4;                // fp32 R, 16-byte aligned rows
    constexpr int LDO = cmax(DK, CP) + EPV;    // W staging rows
    constexpr int LDP = CP + EPV;              // P staging rows (inside the R area)
    constexpr int LDX = C / 2 + 1;             // temporary of the block doubling
    // LDS regions, reused across phases:
    //   Y: K rows -> V^T -> W staging        Z: K^T (whole kernel)
    //   X: V rows -> A and R (P staged inside the R area before R is formed)
    constexpr int RY = cmax(cmax(C * LDK, DV * LDT), C * LDO);
    constexpr int RZ = DK * LDT;
    constexpr int RX = cmax(C * LDA + C * LDR, (C * LDV * (int)sizeof(E) + 3) / 4);
    constexpr int NG = NT * (NT + 1) / 2;      // lower-triangular 16x16 tiles (incl. diagonal)
    constexpr int GPW = (2 * NG + 3) / 4;      // Gram tiles held per wave
    static_assert(C * LDP * (int)sizeof(E) <= C * LDR * 4, "P staging must fit in the R area");

    __shared__ __align__(16) E sm_y[RY];
    __shared__ __align__(16) E sm_z[RZ];
    __shared__ __align__(16) float sm_x[RX];
    __shared__ float sm_t[(C / 2 > 16 ? C / 2 : 16) * LDX];
    __shared__ float sm_gam[C];
    __shared__ float sm_beta[CP];
    __shared__ float sm_bg[CP];   // beta * Gamma

    const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int T = p.T, Hk = p.Hk, Hv = p.Hv, N = p.N;
    const int grp = Hv / Hk;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, kq = (lane >> 4) * KPL, rq = (lane >> 4) * 4;

    const E* kg = reinterpret_cast<const E*>(p.k) + ((size_t)b * T + t0) * Hk * DK + (size_t)hk * DK;
    const E* qg = reinterpret_cast<const E*>(p.q) + ((size_t)b * T + t0) * Hk * DK + (size_t)hk * DK;
    const size_t rsk = (size_t)Hk * DK, rsv = (size_t)Hv * DV;

    E* Ks = sm_y;
    E* KsT = sm_z;
    E* VsT = sm_y;
    E* Os = sm_y;
    E* Vs = reinterpret_cast<E*>(sm_x);
    float* sA = sm_x;
    float* sR = sm_x + C * LDA;
    E* Ps = reinterpret_cast<E*>(sR);

    // -- K rows (rows >= n are zero) -----------------------------------------------------------
    constexpr int VK = DK / EPV;
    for (int idx = tid; idx < C * VK; idx += kThreads) {
        const int r = idx / VK, cv = idx % VK;
        uint4 a = {0u, 0u, 0u, 0u};
        if (r < n) a = *reinterpret_cast<const uint4*>(kg + r * rsk + cv * EPV);
        *reinterpret_cast<uint4*>(Ks + r * LDK + cv * EPV) = a;
    }
    lds_barrier();

    // -- K^T (token-contiguous, zero tokens up to CP); adjacent lanes read adjacent columns -----
    for (int idx = tid; idx < DK * (CP / EPV); idx += kThreads) {
        const int d = idx % DK, s0 = (idx / DK) * EPV;
        uint4 raw;
        E* tmp = reinterpret_cast<E*>(&raw);
#pragma unroll
        for (int e = 0; e < EPV; ++e) tmp[e] = (s0 + e < C) ? Ks[(s0 + e) * LDK + d] : X::from_f(0.f);
        *reinterpret_cast<uint4*>(KsT + d * LDT + s0) = raw;
    }

    // -- Gram tiles on MFMA, kept in registers across the value heads -------------------------
    //   ti <  NG: K K^T, D[r][s]  (r in tile tm, s in tile tn)
    //   ti >= NG: K Q^T, D[s][r]  (s in tile tn, r in tile tm), i.e. P^T before masking;
    //             the Q rows come straight from global memory.
    f32x4 G[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int ti = wave + 4 * gi;
        G[gi] = zero4();
        if (ti < 2 * NG) {
            const bool isq = ti >= NG;
            int tm, tn;
            lower_tile(isq ? ti - NG : ti, tm, tn);
            const E* ar = Ks + ((isq ? tn : tm) * 16 + rl) * LDK + kq;
            f32x4 acc = zero4();
            if (!isq) {
                const E* br = Ks + (tn * 16 + rl) * LDK + kq;
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) acc = X::mma(X::ld(ar + kb * KB), X::ld(br + kb * KB), acc);
            } else {
                const int rq_row = tm * 16 + rl;
                const E* br = qg + (size_t)rq_row * rsk + kq;
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) {
                    const typename X::frag bq = (rq_row < n) ? X::ld(br + kb * KB) : X::zero();
                    acc = X::mma(X::ld(ar + kb * KB), bq, acc);
                }
            }
            G[gi] = acc;
        }
    }
    lds_barrier();   // K^T complete; K rows no longer needed

    // -- K^T fragments for the scan (written once per key head) -------------------------------
    {
        E* KTg = reinterpret_cast<E*>(p.KT) + (((size_t)b * Hk + hk) * N + c) * S::KT_PER_CHUNK;
        for (int f = wave; f < (DK / 16) * NKC; f += kThreads / 64) {
            const int dt = f / NKC, kb = f % NKC;
            store_frag(KTg + ((size_t)f * 64 + lane) * KPL, KsT + (dt * 16 + rl) * LDT + kb * KB + kq);
        }
    }

    for (int hh = 0; hh < grp; ++hh) {
        const int h = hk * grp + hh;
        const size_t bh = (size_t)b * Hv + h;

        // -- gates: running log-gate over the chunk, beta, beta * Gamma; V rows ----------------
        if (wave == 0) {
            const size_t gi = ((size_t)b * T + t0 + lane) * Hv + h;
            float x = (lane < n) ? p.g[gi] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            const float bt = (lane < n) ? p.beta[gi] : 0.f;
            if (lane < C) sm_gam[lane] = x;
            if (lane < CP) {
                sm_beta[lane] = bt;
                sm_bg[lane] = bt * expf(x);
            }
        }
        const E* vg = reinterpret_cast<const E*>(p.v) + ((size_t)b * T + t0) * rsv + (size_t)h * DV;
        constexpr int VV = DV / EPV;
        for (int idx = tid; idx < C * VV; idx += kThreads) {
            const int r = idx / VV, cv = idx % VV;
            uint4 a = {0u, 0u, 0u, 0u};
            if (r < n) a = *reinterpret_cast<const uint4*>(vg + r * rsv + cv * EPV);
            *reinterpret_cast<uint4*>(Vs + r * LDV + cv * EPV) = a;
        }
        lds_barrier();
        for (int idx = tid; idx < DV * (CP / EPV); idx += kThreads) {
            const int d = idx % DV, s0 = (idx / DV) * EPV;
            uint4 raw;
            E* tmp = reinterpret_cast<E*>(&raw);
#pragma unroll
            for (int e = 0; e < EPV; ++e) tmp[e] = (s0 + e < C) ? Vs[(s0 + e) * LDV + d] : X::from_f(0.f);
            *reinterpret_cast<uint4*>(VsT + d * LDT + s0) = raw;
        }
        lds_barrier();   // V rows consumed: the X area now holds A and R

        // -- masks: A (fp32) and P (staged as P[r][s] in the R area) ---------------------------
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int ti = wave + 4 * gi;
            if (ti < 2 * NG) {
                const bool isq = ti >= NG;
                int tm, tn;
                lower_tile(isq ? ti - NG : ti, tm, tn);
                if (!isq) {
                    const int s = tn * 16 + rl;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = tm * 16 + rq + j;
                        sA[r * LDA + s] = (s < r) ? sm_beta[r] * expf(sm_gam[r] - sm_gam[s]) * G[gi][j] : 0.f;
                    }
                } else {
                    const int r = tm * 16 + rl;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int s = tn * 16 + rq + j;
                        const float val = (s <= r) ? expf(sm_gam[r] - sm_gam[s]) * G[gi][j] : 0.f;
                        Ps[r * LDP + s] = X::from_f(val);
                    }
                }
            }
        }
        for (int e = tid; e < C * CP; e += kThreads) {   // tiles above the diagonal are zero
            const int r = e / CP, s = e % CP;
            if ((s >> 4) > (r >> 4)) {
                if (s < C) sA[r * LDA + s] = 0.f;
                Ps[r * LDP + s] = X::from_f(0.f);
            }
        }
        lds_barrier();
        {
            E* Pg = reinterpret_cast<E*>(p.P) + (bh * N + c) * S::P_PER_CHUNK;
            for (int f = wave; f < NT * NKC; f += kThreads / 64) {
                const int m = f / NKC, kb = f % NKC;
                store_frag(Pg + ((size_t)f * 64 + lane) * KPL, Ps + (m * 16 + rl) * LDP + kb * KB + kq);
            }
        }
        lds_barrier();   // P staging consumed: the R area is free

        // -- R = (I + A)^-1: 16x16 diagonal blocks by substitution, then block doubling ------
        if (tid < NT * 16) {
            const int base = (tid >> 4) * 16, j = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s -= sA[(base + r) * LDA + base + m] * x[m];
                x[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sR[(base + r) * LDR + base + j] = x[r];
        }
        for (int e = tid; e < C * CP; e += kThreads) {
            const int r = e / CP, s = e % CP;
            if ((s >> 4) > (r >> 4)) sR[r * LDR + s] = 0.f;
        }
        lds_barrier();
        // [[R11, 0], [R21, R22]] with R21 = -R22 A21 R11, for block sizes 16, 32, ... < C
        for (int bs = 16; bs < C; bs *= 2) {
            const int npair = C / (2 * bs), tpb = bs / 16, tiles = npair * tpb * tpb;
            for (int t = wave; t < tiles; t += kThreads / 64) {
                const int pr = t / (tpb * tpb), ti = (t % (tpb * tpb)) / tpb, tj = t % tpb;
                const int lo = pr * 2 * bs, hi = lo + bs;
                const f32x4 acc = mma_tile_f32(sA + (hi + ti * 16) * LDA + lo, LDA,
                                               sR + lo * LDR + lo + tj * 16, LDR, bs, zero4(), lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) sm_t[(pr * bs + ti * 16 + rq + j) * LDX + tj * 16 + rl] = acc[j];
            }
            lds_barrier();
            for (int t = wave; t < tiles; t += kThreads / 64) {
                const int pr = t / (tpb * tpb), ti = (t % (tpb * tpb)) / tpb, tj = t % tpb;
                const int lo = pr * 2 * bs, hi = lo + bs;
                const f32x4 acc = mma_tile_f32(sR + (hi + ti * 16) * LDR + hi, LDR,
                                               sm_t + (pr * bs) * LDX + tj * 16, LDX, bs, zero4(), lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) sR[(hi + ti * 16 + rq + j) * LDR + lo + tj * 16 + rl] = -acc[j];
            }
            lds_barrier();
        }

        // -- Ut = R diag(beta) V as accumulator tiles, then W = R diag(beta Gamma) K staged ----
        auto rtile = [&](int tm, const float* scale, const E* bsrc) {
            const float* arow = sR + (tm * 16 + rl) * LDR + kq;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) {
                float av[KPL];
#pragma unroll
                for (int e = 0; e < KPL; ++e) av[e] = arow[kb * KB + e] * scale[kb * KB + kq + e];
                acc = X::mma(X::ld_f(av), X::ld(bsrc + kb * KB), acc);
            }
            return acc;
        };
        {
            E* Ug = reinterpret_cast<E*>(p.Ut) + (bh * N + c) * S::UT_PER_CHUNK;
            for (int ti = wave; ti < NT * (DV / 16); ti += kThreads / 64) {
                const int tm = ti / (DV / 16), tn = ti % (DV / 16);
                const f32x4 acc = rtile(tm, sm_beta, VsT + (tn * 16 + rl) * LDT + kq);
                E ov[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = X::from_f(acc[j]);
                store4(Ug + (((size_t)tn * NT + tm) * 64 + lane) * 4, ov);
            }
        }
        lds_barrier();   // V^T consumed: Y becomes the W staging area
        for (int ti = wave; ti < NT * (DK / 16); ti += kThreads / 64) {
            const int tm = ti / (DK / 16), tn = ti % (DK / 16);
            const f32x4 acc = rtile(tm, sm_bg, KsT + (tn * 16 + rl) * LDT + kq);
#pragma unroll
            for (int j = 0; j < 4; ++j) Os[(tm * 16 + rq + j) * LDO + tn * 16 + rl] = X::from_f(acc[j]);
        }
        lds_barrier();
        {
            E* Wg = reinterpret_cast<E*>(p.W) + (bh * N + c) * S::W_PER_CHUNK;
            for (int f = wave; f < NT * NKD; f += kThreads / 64) {
                const int m = f / NKD, kb = f % NKD;
                store_frag(Wg + ((size_t)f * 64 + lane) * KPL, Os + (m * 16 + rl) * LDO + kb * KB + kq);
            }
        }
        if (tid < C) {   // gate factors for the scan: exp(gamma_r), then exp(gamma_last - gamma_r)
            float* gf = p.gam + (bh * N + c) * 2 * C;
            gf[tid] = expf(sm_gam[tid]);
            gf[C + tid] = expf(sm_gam[C - 1] - sm_gam[tid]);
        }
        lds_barrier();   // staging, V buffers and gates are reused by the next value head
    }
}

// ------------------------------------------------------------------------------------
// Kernel 2: chunks in order; fp32 state slice in accumulator registers.
//
// Eight waves per workgroup in two roles.  Chain waves 0..3 carry the recurrence:
// U = Ut - W S^T for their 16-token tile, then S^T <- Gamma_n S^T + K^T (e * U) for their
// state tiles.  Output waves 4..7 compute O = Gamma (Q S^T) + P U for their token tile one
// barrier behind, from a double-buffered copy of the state, so the output products stay off
// the chain.  Each role prefetches its own operands NB chunks ahead into registers.
// SPLIT: feed the state to W S^T as a bf16 hi + lo pair (two MFMAs) so the delta U sees
// the fp32 state to ~16 bits instead of 8.
// ------------------------------------------------------------------------------------
constexpr int kScanThreads = 512;
// operand sets in flight per wave: chain waves are on the critical path and prefetch
// deeper; fp32 operands take four times the registers of bf16 ones
template <typename E> struct ScanDepth;
template <> struct ScanDepth<bf16_t> { static constexpr int chain = 3, output = 2; };
template <> struct ScanDepth<float> { static constexpr int chain = 2, output = 1; };

template <typename E, int DK, int C, int TPW>
struct ChainOperands {
    using X = Elem<E>;
    typedef typename X::frag frag;
    static constexpr int NKD = DK / X::KB;
    static constexpr int NKC = (C + X::KB - 1) / X::KB;
    frag w[NKD];
    frag kt[TPW][NKC];
    E ut[4];
    f32x4 e;      // exp(gamma_last - gamma_r) for this lane's four token rows
    float gn;     // exp(gamma_last)
};

template <typename E, int DK, int C>
struct OutputOperands {
    using X = Elem<E>;
    typedef typename X::frag frag;
    static constexpr int NKD = DK / X::KB;
    static constexpr int NKC = (C + X::KB - 1) / X::KB;
    frag q[NKD];
    frag p[NKC];
    f32x4 gr;     // exp(gamma_r) for this lane's four token rows
};

template <typename E, int DK, int DV, int C, bool SPLIT>
__global__ __launch_bounds__(kScanThreads) void inter_chunk_kernel(PrefillParams p) {
    using Sh = PrefillShape<E, DK, DV, C>;
    using X = Elem<E>;
    typedef typename X::frag frag;
    constexpr int KB = Sh::KB, KPL = Sh::KPL, NT = Sh::NT, NKD = Sh::NKD, NKC = Sh::NKC;
    constexpr int EPV = 16 / (int)sizeof(E);
    constexpr int DT = DK / 16;
    constexpr int TPW = (DT + 3) / 4;
    constexpr int LDS_ = DK + EPV;
    constexpr int CP = NKC * KB;
    constexpr int LDU = CP + EPV;
    constexpr int NSLICE = DV / 16;
    constexpr int NBC = ScanDepth<E>::chain, NBO = ScanDepth<E>::output;
    typedef ChainOperands<E, DK, C, TPW> COps;
    typedef OutputOperands<E, DK, C> OOps;

    __shared__ __align__(16) E Sb[2][16 * LDS_];              // state slice, hi part, 2 buffers
    __shared__ __align__(16) E Sl[2][SPLIT ? 16 * LDS_ : EPV];  // lo part
    __shared__ __align__(16) E UT[16 * LDU];                   // U^T        (for P U)
    __shared__ __align__(16) E UsT[16 * LDU];                  // (e * U)^T  (for the update)

    // XCD-aware placement: consecutive workgroups go to different XCDs; place the slices of
    // one head on the same XCD so they share its L2 for the head's chunk operands.
    const int total = p.B * p.Hv * NSLICE;
    int unit = blockIdx.x;
    if ((total & 7) == 0) unit = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int slice = unit % NSLICE;
    const int bh = unit / NSLICE;
    const int h = bh % p.Hv, b = bh / p.Hv;
    const int T = p.T, Hk = p.Hk, Hv = p.Hv, N = p.N;
    const int hk = h / (Hv / Hk);
    const int i0 = slice * 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int rl = lane & 15, kq = (lane >> 4) * KPL, rq = (lane >> 4) * 4;
    const bool chain = wave < 4;
    const int w4 = wave & 3;
    const bool has_tile = w4 < NT;
    const int m = w4 % NT;           // token tile (duplicate for waves past the chunk's tiles)
    const int Nf = T / C;            // full chunks; a partial last chunk takes the tail path
    std::integral_constant<bool, false> full;
    std::integral_constant<bool, true> tail;

    const float* gates = p.gam + (size_t)bh * N * 2 * C;   // per chunk: exp(gamma) then exp(gl - gamma)

    for (int e = tid; e < 16 * LDU; e += kScanThreads) {   // columns past the chunk read as zero
        UT[e] = X::from_f(0.f);
        UsT[e] = X::from_f(0.f);
    }

    if (chain) {
        const E* Wg = reinterpret_cast<const E*>(p.W) + (size_t)bh * N * Sh::W_PER_CHUNK;
        const E* Ug = reinterpret_cast<const E*>(p.Ut) + (size_t)bh * N * Sh::UT_PER_CHUNK;
        const E* KTg = reinterpret_cast<const E*>(p.KT) + ((size_t)b * Hk + hk) * N * Sh::KT_PER_CHUNK;

        auto fetch = [&](COps& op, int c) {
            const float* gc = gates + (size_t)c * 2 * C;
            op.gn = gc[C - 1];
            op.e = *reinterpret_cast<const f32x4*>(gc + C + m * 16 + rq);
            const E* wsrc = Wg + (size_t)c * Sh::W_PER_CHUNK + (size_t)m * NKD * Sh::FRAG + lane * KPL;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) op.w[kb] = X::ld(wsrc + kb * Sh::FRAG);
            const E* usrc = Ug + (size_t)c * Sh::UT_PER_CHUNK + (((size_t)slice * NT + m) * 64 + lane) * 4;
            if (sizeof(E) == 2) *reinterpret_cast<uint2*>(op.ut) = *reinterpret_cast<const uint2*>(usrc);
            else *reinterpret_cast<uint4*>(op.ut) = *reinterpret_cast<const uint4*>(usrc);
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                const int dt = min(w4 + 4 * tw, DT - 1);
                const E* ksrc = KTg + (size_t)c * Sh::KT_PER_CHUNK + ((size_t)dt * NKC * 64 + lane) * KPL;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) op.kt[tw][kb] = X::ld(ksrc + kb * Sh::FRAG);
            }
        };

        // state slice: S^T tiles (rows = dk index, cols = the 16 state rows of this slice)
        f32x4 St[TPW];
        const size_t sbase = ((size_t)bh * DV + i0 + rl) * DK;
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int dt = w4 + 4 * tw;
            St[tw] = zero4();
            if (dt < DT && p.state_in) {
                const float4 s4 = *reinterpret_cast<const float4*>(p.state_in + sbase + dt * 16 + rq);
                St[tw][0] = s4.x; St[tw][1] = s4.y; St[tw][2] = s4.z; St[tw][3] = s4.w;
            }
        }
        auto publish = [&](int buf) {
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                const int dt = w4 + 4 * tw;
                if (dt < DT) {
                    E hi[4], lo[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        hi[j] = X::from_f(St[tw][j]);
                        lo[j] = X::from_f(St[tw][j] - X::to_f(hi[j]));
                    }
                    store4(&Sb[buf][rl * LDS_ + dt * 16 + rq], hi);
                    if (SPLIT) store4(&Sl[buf][rl * LDS_ + dt * 16 + rq], lo);
                }
            }
        };
        auto step = [&](const COps& op, int c) {
            const int cur = c & 1;
            if (has_tile) {
                const E* sr = &Sb[cur][rl * LDS_ + kq];
                const E* sl = &Sl[cur][SPLIT ? rl * LDS_ + kq : 0];
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) {
                    acc = X::mma(op.w[kb], X::ld(sr + kb * KB), acc);
                    if (SPLIT) acc = X::mma(op.w[kb], X::ld(sl + kb * KB), acc);
                }
                E u[4], us[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float uj = X::to_f(op.ut[j]) - acc[j];
                    u[j] = X::from_f(uj);
                    us[j] = X::from_f(uj * op.e[j]);
                }
                store4(UT + rl * LDU + m * 16 + rq, u);
                store4(UsT + rl * LDU + m * 16 + rq, us);
            }
            lds_barrier();   // (B1) U complete; chunk c's slice was read from buffer cur
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                const int dt = w4 + 4 * tw;
                if (dt < DT) {
                    f32x4 acc = St[tw] * op.gn;
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        acc = X::mma(op.kt[tw][kb], X::ld(UsT + rl * LDU + kb * KB + kq), acc);
                    St[tw] = acc;
                }
            }
            publish(cur ^ 1);
            lds_barrier();   // (B2) next slice published; output waves are done with U
        };

        publish(0);
        COps op[NBC];
#pragma unroll
        for (int j = 0; j < NBC; ++j) fetch(op[j], min(j, N - 1));
        lds_barrier();
        int c = 0;
        for (; c + NBC <= N; c += NBC) {
#pragma unroll
            for (int j = 0; j < NBC; ++j) {
                step(op[j], c + j);
                fetch(op[j], min(c + j + NBC, N - 1));
            }
        }
#pragma unroll
        for (int j = 0; j < NBC; ++j)
            if (c + j < N) step(op[j], c + j);

#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int dt = w4 + 4 * tw;
            if (dt < DT) {
                float4 s4;
                s4.x = St[tw][0]; s4.y = St[tw][1]; s4.z = St[tw][2]; s4.w = St[tw][3];
                *reinterpret_cast<float4*>(p.state_out + sbase + dt * 16 + rq) = s4;
            }
        }
    } else {
        const E* Pg = reinterpret_cast<const E*>(p.P) + (size_t)bh * N * Sh::P_PER_CHUNK;
        const E* qg = reinterpret_cast<const E*>(p.q) + (size_t)hk * DK;
        E* og = reinterpret_cast<E*>(p.o) + (size_t)h * DV + i0;

        auto fetch = [&](OOps& op, int c) {
            const int t0 = c * C;
            op.gr = *reinterpret_cast<const f32x4*>(gates + (size_t)c * 2 * C + m * 16 + rq);
            const int tq = t0 + m * 16 + rl;
            const E* qsrc = qg + ((size_t)b * T + min(tq, T - 1)) * Hk * DK + kq;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) op.q[kb] = X::ld(qsrc + kb * KB);   // rows past T: zeroed in the tail
            const E* psrc = Pg + (size_t)c * Sh::P_PER_CHUNK + (size_t)m * NKC * Sh::FRAG + lane * KPL;
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) op.p[kb] = X::ld(psrc + kb * Sh::FRAG);
        };
        auto step = [&](const OOps& op, int c, auto tailtag) {
            constexpr bool TAIL = decltype(tailtag)::value;
            const int t0 = c * C;
            lds_barrier();   // (B1) U of chunk c is in LDS; buffer (c & 1) holds chunk c's slice
            if (has_tile) {
                const E* sr = &Sb[c & 1][rl * LDS_ + kq];
                const bool qok = !TAIL || (t0 + m * 16 + rl < T);
                f32x4 accq = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb)
                    accq = X::mma(TAIL ? X::keep_if(op.q[kb], qok) : op.q[kb], X::ld(sr + kb * KB), accq);
                f32x4 acc = accq * op.gr;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) acc = X::mma(op.p[kb], X::ld(UT + rl * LDU + kb * KB + kq), acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = t0 + m * 16 + rq + j;
                    if (!TAIL || t < T) og[((size_t)b * T + t) * Hv * DV + rl] = X::from_f(acc[j]);
                }
            }
            lds_barrier();   // (B2)
        };

        OOps op[NBO];
#pragma unroll
        for (int j = 0; j < NBO; ++j) fetch(op[j], min(j, N - 1));
        lds_barrier();
        int c = 0;
        for (; c + NBO <= Nf; c += NBO) {
#pragma unroll
            for (int j = 0; j < NBO; ++j) {
                step(op[j], c + j, full);
                fetch(op[j], min(c + j + NBO, N - 1));
            }
        }
#pragma unroll
        for (int j = 0; j < NBO; ++j) {
            if (c + j < Nf) step(op[j], c + j, full);
            else if (c + j < N) step(op[j], c + j, tail);
        }
    }
}

// stage bit 1: intra-chunk kernel; bit 2: inter-chunk kernel.
template <typename E, int DK, int DV, int C>
inline hipError_t launch_prefill(const PrefillParams& p, int stages, hipStream_t stream) {
    if (stages & 1) {
        dim3 g1(p.N, p.Hk, p.B);
        intra_chunk_kernel<E, DK, DV, C><<<g1, kThreads, 0, stream>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & 2) {
        dim3 g2(p.B * p.Hv * (DV / 16));
        inter_chunk_kernel<E, DK, DV, C, sizeof(E) == 2><<<g2, kScanThreads, 0, stream>>>(p);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace gdn
