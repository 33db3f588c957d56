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
// Kernel 1 (intra_chunk_kernel), one workgroup per (batch, value head, chunk), fully
// parallel: stages K, Q in LDS, forms both Gram tiles on MFMA, writes P, inverts
// (I + A) in fp32 by 16x16 diagonal blocks plus block back-substitution, and forms W and
// Ut on MFMA.  W, Ut, P, the within-chunk gamma and a transposed copy of each chunk's K
// go to the workspace.
//
// Kernel 2 (inter_chunk_kernel), one workgroup per (batch, value head, 16 state rows):
// rows of S evolve independently (each needs only its own entries of v), so a head's
// state is split into 16-row slices that never talk to each other.  The fp32 slice
// lives in MFMA accumulator registers for the whole scan and is written back once at
// the end ("Keep the recurrent state on chip": load the state once, carry it through
// the scan, write it after).  Per chunk: U = Ut - W S^T and Q S^T (tokens x rows), the
// output tile, then S^T <- Gamma S^T + K^T (decayed U).
#pragma once

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
    void* W;     // [B][Hv][Tp][DK]     E
    void* Ut;    // [B][Hv][Tp][DV]     E
    void* P;     // [B][Hv][Tp][C]      E   (row r of chunk c at c*C + r)
    void* KT;    // [B][Hk][N][DK][C]   E   (chunk-local transpose of K)
    float* gam;  // [B][Hv][Tp]             (within-chunk running log-gate)
    int B, T, Hk, Hv, N;  // N = number of chunks, Tp = N * C
};

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------
// Kernel 1: per-chunk, state-independent blocks.
// ------------------------------------------------------------------------------------
template <typename E, int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void intra_chunk_kernel(PrefillParams p) {
    using X = Elem<E>;
    constexpr int KB = X::KB, KPL = X::KPL;
    constexpr int EPV = 16 / (int)sizeof(E);  // elements per 16-byte vector
    constexpr int LDK = DK + EPV;             // row stride of K / Q tiles (elements)
    constexpr int LDC = C + EPV;              // row stride of token-contiguous tiles
    constexpr int LDA = C + 1;                // fp32 A
    constexpr int LDR = C + 4;                // fp32 R (rows 16-byte aligned)
    constexpr int NT = C / 16;                // 16-token tiles per chunk
    constexpr int PH1 = 2 * C * LDK;
    constexpr int PH4 = (DK + DV) * LDC;
    constexpr int UNION = PH1 > PH4 ? PH1 : PH4;
    constexpr int NX = NT > 1 ? NT - 1 : 1;

    __shared__ __align__(16) E sm_u[UNION];
    __shared__ float sm_A[C * LDA];
    __shared__ __align__(16) float sm_R[C * LDR];
    __shared__ float sm_X[NX * 16 * 17];
    __shared__ float sm_gam[C];
    __shared__ float sm_beta[C];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int T = p.T, Hk = p.Hk, Hv = p.Hv;
    const int hk = h / (Hv / Hk);
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t Tp = (size_t)p.N * C;

    const E* kg = reinterpret_cast<const E*>(p.k) + ((size_t)b * T + t0) * Hk * DK + (size_t)hk * DK;
    const E* qg = reinterpret_cast<const E*>(p.q) + ((size_t)b * T + t0) * Hk * DK + (size_t)hk * DK;
    const E* vg = reinterpret_cast<const E*>(p.v) + ((size_t)b * T + t0) * Hv * DV + (size_t)h * DV;
    const size_t rsk = (size_t)Hk * DK, rsv = (size_t)Hv * DV;

    E* Ks = sm_u;
    E* Qs = sm_u + C * LDK;

    // -- stage K, Q (rows >= n are zero) and the gates ----------------------------------
    constexpr int VK = DK / EPV;
    for (int idx = tid; idx < C * VK; idx += kThreads) {
        const int r = idx / VK, cv = idx % VK;
        uint4 a = {0u, 0u, 0u, 0u}, bq = {0u, 0u, 0u, 0u};
        if (r < n) {
            a = *reinterpret_cast<const uint4*>(kg + r * rsk + cv * EPV);
            bq = *reinterpret_cast<const uint4*>(qg + r * rsk + cv * EPV);
        }
        *reinterpret_cast<uint4*>(Ks + r * LDK + cv * EPV) = a;
        *reinterpret_cast<uint4*>(Qs + r * LDK + cv * EPV) = bq;
    }
    if (wave == 0) {
        const size_t gi = ((size_t)b * T + t0 + lane) * Hv + h;
        float x = (lane < n) ? p.g[gi] : 0.f;
        // inclusive running sum over the chunk (wave-wide scan)
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane < C) {
            sm_gam[lane] = x;
            sm_beta[lane] = (lane < n) ? p.beta[gi] : 0.f;
        }
    }
    __syncthreads();

    // -- Gram tiles on MFMA: A (masked K K^T) to LDS, P (masked Q K^T) to workspace -------
    E* Pg = reinterpret_cast<E*>(p.P) + (((size_t)b * Hv + h) * Tp + t0) * C;
    {
        const int rl = lane & 15, kq = (lane >> 4) * KPL;
        for (int ti = wave; ti < 2 * NT * NT; ti += kThreads / 64) {
            const bool isq = ti >= NT * NT;
            const int tt = isq ? ti - NT * NT : ti;
            const int tm = tt / NT, tn = tt % NT;
            f32x4 acc = zero4();
            if (tn <= tm) {
                const E* ar = (isq ? Qs : Ks) + (tm * 16 + rl) * LDK + kq;
                const E* br = Ks + (tn * 16 + rl) * LDK + kq;
#pragma unroll
                for (int kb = 0; kb < DK; kb += KB) acc = X::mma(X::ld(ar + kb), X::ld(br + kb), acc);
            }
            const int s = tn * 16 + rl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = tm * 16 + (lane >> 4) * 4 + j;
                if (!isq) {
                    sm_A[r * LDA + s] = (s < r) ? sm_beta[r] * expf(sm_gam[r] - sm_gam[s]) * acc[j] : 0.f;
                } else {
                    const float val = (s <= r) ? expf(sm_gam[r] - sm_gam[s]) * acc[j] : 0.f;
                    Pg[(size_t)r * C + s] = X::from_f(val);
                }
            }
        }
    }
    __syncthreads();

    // -- R = (I + A)^-1: diagonal 16x16 blocks by forward substitution ---------------------
    if (tid < NT * 16) {
        const int base = (tid >> 4) * 16, j = tid & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) s -= sm_A[(base + r) * LDA + base + m] * x[m];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm_R[(base + r) * LDR + base + j] = x[r];
    }
    // zero the strictly-upper blocks of R
    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, s = e % C;
        if ((s >> 4) > (r >> 4)) sm_R[r * LDR + s] = 0.f;
    }
    __syncthreads();
    // off-diagonal blocks, by distance d from the diagonal:
    //   R_ij = -R_ii * sum_{j <= m < i} A_im R_mj
    for (int d = 1; d < NT; ++d) {
        const int nblk = NT - d;
        for (int e = tid; e < nblk * 256; e += kThreads) {
            const int jb = e >> 8, rr = (e & 255) >> 4, cc = e & 15, ib = jb + d;
            float s = 0.f;
            for (int m = jb * 16; m < ib * 16; ++m)
                s += sm_A[(ib * 16 + rr) * LDA + m] * sm_R[m * LDR + jb * 16 + cc];
            sm_X[jb * 272 + rr * 17 + cc] = s;
        }
        __syncthreads();
        for (int e = tid; e < nblk * 256; e += kThreads) {
            const int jb = e >> 8, rr = (e & 255) >> 4, cc = e & 15, ib = jb + d;
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m)
                s += sm_R[(ib * 16 + rr) * LDR + ib * 16 + m] * sm_X[jb * 272 + m * 17 + cc];
            sm_R[(ib * 16 + rr) * LDR + jb * 16 + cc] = -s;
        }
        __syncthreads();
    }

    // -- token-contiguous (transposed) operands: (beta Gamma K)^T and (beta V)^T ----------
    E* KbT = sm_u;            // [DK][LDC]
    E* VbT = sm_u + DK * LDC;  // [DV][LDC]
    E* KTg = reinterpret_cast<E*>(p.KT) + (((size_t)b * Hk + hk) * p.N + c) * DK * C;
    const bool write_kt = (h % (Hv / Hk)) == 0;
    for (int idx = tid; idx < C * VK; idx += kThreads) {
        const int r = idx / VK, cv = idx % VK;
        uint4 raw = {0u, 0u, 0u, 0u};
        if (r < n) raw = *reinterpret_cast<const uint4*>(kg + r * rsk + cv * EPV);
        const E* tmp = reinterpret_cast<const E*>(&raw);
        const float sc = sm_beta[r] * expf(sm_gam[r]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            KbT[(cv * EPV + e) * LDC + r] = X::from_f(X::to_f(tmp[e]) * sc);
            if (write_kt) KTg[(size_t)(cv * EPV + e) * C + r] = tmp[e];
        }
    }
    constexpr int VV = DV / EPV;
    for (int idx = tid; idx < C * VV; idx += kThreads) {
        const int r = idx / VV, cv = idx % VV;
        uint4 raw = {0u, 0u, 0u, 0u};
        if (r < n) raw = *reinterpret_cast<const uint4*>(vg + r * rsv + cv * EPV);
        const E* tmp = reinterpret_cast<const E*>(&raw);
        const float sc = sm_beta[r];
#pragma unroll
        for (int e = 0; e < EPV; ++e) VbT[(cv * EPV + e) * LDC + r] = X::from_f(X::to_f(tmp[e]) * sc);
    }
    __syncthreads();

    // -- W = R (beta Gamma K), Ut = R (beta V) on MFMA -------------------------------------
    E* Wg = reinterpret_cast<E*>(p.W) + (((size_t)b * Hv + h) * Tp + t0) * DK;
    E* Ug = reinterpret_cast<E*>(p.Ut) + (((size_t)b * Hv + h) * Tp + t0) * DV;
    {
        constexpr int TW = NT * (DK / 16), TU = NT * (DV / 16);
        const int rl = lane & 15, kq = (lane >> 4) * KPL;
        for (int ti = wave; ti < TW + TU; ti += kThreads / 64) {
            const bool isu = ti >= TW;
            const int tt = isu ? ti - TW : ti;
            const int nd = isu ? DV / 16 : DK / 16;
            const int tm = tt / nd, tn = tt % nd;
            const E* BT = isu ? VbT : KbT;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < C; kb += KB) {
                const int k0 = kb + kq;
                const typename X::frag a = (k0 < C) ? X::ld_f(sm_R + (tm * 16 + rl) * LDR + k0) : X::zero();
                const typename X::frag bb = (k0 < C) ? X::ld(BT + (tn * 16 + rl) * LDC + k0) : X::zero();
                acc = X::mma(a, bb, acc);
            }
            E* out = isu ? Ug : Wg;
            const int D = isu ? DV : DK;
            const int col = tn * 16 + rl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = tm * 16 + (lane >> 4) * 4 + j;
                out[(size_t)r * D + col] = X::from_f(acc[j]);
            }
        }
    }
    if (tid < C) p.gam[((size_t)b * Hv + h) * Tp + t0 + tid] = sm_gam[tid];
}

// ------------------------------------------------------------------------------------
// Kernel 2: chunks in order; fp32 state slice in accumulator registers.
// SPLIT: feed the state to W S^T as a bf16 hi + lo pair (two MFMAs) so the delta U
// sees the fp32 state to ~16 bits instead of 8.
// ------------------------------------------------------------------------------------
template <typename E, int DK, int DV, int C, bool SPLIT>
__global__ __launch_bounds__(kThreads) void inter_chunk_kernel(PrefillParams p) {
    using X = Elem<E>;
    typedef typename X::frag frag;
    constexpr int KB = X::KB, KPL = X::KPL;
    constexpr int EPV = 16 / (int)sizeof(E);
    constexpr int NT = C / 16;
    constexpr int DT = DK / 16;
    constexpr int TPW = (DT + 3) / 4;
    constexpr int LDS_ = DK + EPV;
    constexpr int LDU = C + EPV;
    constexpr int NSLICE = DV / 16;

    __shared__ __align__(16) E Sb[16 * LDS_];
    __shared__ __align__(16) E Sl[SPLIT ? 16 * LDS_ : EPV];
    __shared__ __align__(16) E UT[16 * LDU];
    __shared__ __align__(16) E UsT[16 * LDU];
    __shared__ float sg[C];

    const int slice = blockIdx.x % NSLICE;
    const int bh = blockIdx.x / NSLICE;
    const int h = bh % p.Hv, b = bh / p.Hv;
    const int T = p.T, Hk = p.Hk, Hv = p.Hv, N = p.N;
    const int hk = h / (Hv / Hk);
    const int i0 = slice * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, kq = (lane >> 4) * KPL, rq = (lane >> 4) * 4;
    const size_t Tp = (size_t)N * C;

    const E* Wg = reinterpret_cast<const E*>(p.W) + ((size_t)b * Hv + h) * Tp * DK;
    const E* Ug = reinterpret_cast<const E*>(p.Ut) + ((size_t)b * Hv + h) * Tp * DV;
    const E* Pg = reinterpret_cast<const E*>(p.P) + ((size_t)b * Hv + h) * Tp * C;
    const E* KTg = reinterpret_cast<const E*>(p.KT) + ((size_t)b * Hk + hk) * N * DK * C;
    const float* gg = p.gam + ((size_t)b * Hv + h) * Tp;
    const E* qg = reinterpret_cast<const E*>(p.q) + (size_t)hk * DK;
    E* og = reinterpret_cast<E*>(p.o) + (size_t)h * DV + i0;

    // state slice: S^T tiles (rows = dk index, cols = the 16 state rows of this slice)
    f32x4 S[TPW];
    const size_t sbase = (((size_t)b * Hv + h) * DV + i0 + rl) * DK;
#pragma unroll
    for (int tw = 0; tw < TPW; ++tw) {
        const int dt = wave + 4 * tw;
        S[tw] = zero4();
        if (dt < DT && p.state_in) {
            const float4 s4 = *reinterpret_cast<const float4*>(p.state_in + sbase + dt * 16 + rq);
            S[tw][0] = s4.x; S[tw][1] = s4.y; S[tw][2] = s4.z; S[tw][3] = s4.w;
        }
    }

    for (int c = 0; c < N; ++c) {
        const int t0 = c * C;
        // (1) publish the state slice in MFMA-operand precision; stage gamma
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int dt = wave + 4 * tw;
            if (dt < DT) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = dt * 16 + rq + j;
                    const E hi = X::from_f(S[tw][j]);
                    Sb[rl * LDS_ + d] = hi;
                    if (SPLIT) Sl[rl * LDS_ + d] = X::from_f(S[tw][j] - X::to_f(hi));
                }
            }
        }
        if (tid < C) sg[tid] = gg[t0 + tid];
        __syncthreads();
        const float glast = sg[C - 1];   // gamma_{n-1} (padded rows repeat it)
        const float Gn = expf(glast);

        // (2) U = Ut - W S^T and Q S^T for this wave's 16-token tile
        f32x4 oq = zero4();
        if (wave < NT) {
            const int m = wave;
            const int tr = t0 + m * 16 + rl;           // token row this lane feeds as A
            const E* wr = Wg + (size_t)(t0 + m * 16 + rl) * DK + kq;
            const E* qr = qg + ((size_t)b * T + tr) * Hk * DK + kq;
            const bool qok = tr < T;
            const E* sr = Sb + rl * LDS_ + kq;
            const E* sl = Sl + rl * LDS_ + kq;
            f32x4 acc = zero4(), accq = zero4();
#pragma unroll
            for (int kb = 0; kb < DK; kb += KB) {
                const frag bs = X::ld(sr + kb);
                const frag aw = X::ld(wr + kb);
                acc = X::mma(aw, bs, acc);
                if (SPLIT) acc = X::mma(aw, X::ld(sl + kb), acc);
                const frag aq = qok ? X::ld(qr + kb) : X::zero();
                accq = X::mma(aq, bs, accq);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = m * 16 + rq + j;
                const float u = X::to_f(Ug[(size_t)(t0 + r) * DV + i0 + rl]) - acc[j];
                UT[rl * LDU + r] = X::from_f(u);
                UsT[rl * LDU + r] = X::from_f(u * expf(glast - sg[r]));
                oq[j] = expf(sg[r]) * accq[j];
            }
        }
        __syncthreads();

        // (3) O = Gamma Q S^T + P U
        if (wave < NT) {
            const int m = wave;
            const E* pr = Pg + (size_t)(t0 + m * 16 + rl) * C;
            f32x4 acc = oq;
#pragma unroll
            for (int kb = 0; kb < C; kb += KB) {
                const int k0 = kb + kq;
                const frag a = (k0 < C) ? X::ld(pr + k0) : X::zero();
                const frag bu = (k0 < C) ? X::ld(UT + rl * LDU + k0) : X::zero();
                acc = X::mma(a, bu, acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + m * 16 + rq + j;
                if (t < T) og[((size_t)b * T + t) * Hv * DV + rl] = X::from_f(acc[j]);
            }
        }

        // (4) S^T <- Gamma_{n-1} S^T + K^T (exp(gamma_{n-1} - gamma) U)
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int dt = wave + 4 * tw;
            if (dt < DT) {
                const E* kr = KTg + ((size_t)c * DK + dt * 16 + rl) * C;
                f32x4 acc = S[tw] * Gn;
#pragma unroll
                for (int kb = 0; kb < C; kb += KB) {
                    const int k0 = kb + kq;
                    const frag a = (k0 < C) ? X::ld(kr + k0) : X::zero();
                    const frag bu = (k0 < C) ? X::ld(UsT + rl * LDU + k0) : X::zero();
                    acc = X::mma(a, bu, acc);
                }
                S[tw] = acc;
            }
        }
    }

#pragma unroll
    for (int tw = 0; tw < TPW; ++tw) {
        const int dt = wave + 4 * tw;
        if (dt < DT) {
            float4 s4;
            s4.x = S[tw][0]; s4.y = S[tw][1]; s4.z = S[tw][2]; s4.w = S[tw][3];
            *reinterpret_cast<float4*>(p.state_out + sbase + dt * 16 + rq) = s4;
        }
    }
}

// stage bit 1: intra-chunk kernel; bit 2: inter-chunk kernel.
template <typename E, int DK, int DV, int C>
inline hipError_t launch_prefill(const PrefillParams& p, int stages, hipStream_t stream) {
    if (stages & 1) {
        dim3 g1(p.N, p.Hv, p.B);
        intra_chunk_kernel<E, DK, DV, C><<<g1, kThreads, 0, stream>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & 2) {
        dim3 g2(p.B * p.Hv * (DV / 16));
        inter_chunk_kernel<E, DK, DV, C, sizeof(E) == 2><<<g2, kThreads, 0, stream>>>(p);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace gdn
