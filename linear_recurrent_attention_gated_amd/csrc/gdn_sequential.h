// gdn_sequential.h -- token-sequential prefill of the gated delta rule: the state held in
// registers for the whole prompt.
//
// "Optimizing on-device inference for Apple Silicon", section "Keep the recurrent state on
// chip": the prefill there scans the tokens directly, each part of the state matrix owned by
// one SIMD group whose lanes split it, loaded into registers once, carried through every
// token with cross-lane reductions instead of shared-memory exchanges, and written back once
// after the last token.  Section "Qwen creates three distinct workload shapes" says whether
// this or the blockwise form is faster depends on the dimensions, the workload and the
// hardware; on gfx950 the blockwise form (gdn_prefill.h) moves the work onto the matrix
// cores and wins for long prompts, this form for short ones (no workspace round trip, one
// launch).
//
// Per token t, for state row i (rows evolve independently):
//   s_k = S_i . k_t,  s_q = S_i . q_t                 (lane-group reductions)
//   delta = beta_t (v_t[i] - a_t s_k),   a_t = exp(g_t)
//   S_i <- a_t S_i + delta k_t
//   o_t[i] = S_i(new) . q_t = a_t s_q + delta (k_t . q_t)
//
// Mapping: a row of dk fp32 values is split over L = 16 consecutive lanes, dk / 16 values per
// lane, so the reductions are four DPP steps on the VALU.  A workgroup holds up to 256 / L
// rows of one value head; each lane keeps its 8 state values in registers for all T tokens.
// The token inputs (its 8 elements of q_t and k_t, v_t[i], g_t, beta_t) are independent of
// the state, so they are loaded U tokens ahead into a second register set while the current
// U tokens are computed.
#pragma once

#include <type_traits>

#include "gdn_device.h"
#include "gdn_prefill.h"

namespace gdn {

// N (8, 4 or 2) consecutive elements of q or k, loaded as one or two vectors
template <typename E, int N> struct VecN;
template <int N> struct VecN<bf16_t, N> {
    static_assert(N == 8 || N == 4 || N == 2, "8, 4 or 2 elements");
    uint32_t w[N / 2];
    __device__ __forceinline__ void load(const bf16_t* p) {
        if constexpr (N == 8) {
            const uint4 u = *reinterpret_cast<const uint4*>(p);
            w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
        } else if constexpr (N == 4) {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            w[0] = u.x; w[1] = u.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        }
    }
    __device__ __forceinline__ void to_f(float (&f)[N]) const {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <int N> struct VecN<float, N> {
    static_assert(N == 8 || N == 4 || N == 2, "8, 4 or 2 elements");
    float f_[N];
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (N == 2) {
            const float2 a = *reinterpret_cast<const float2*>(p);
            f_[0] = a.x; f_[1] = a.y;
        } else {
#pragma unroll
            for (int i = 0; i < N / 4; ++i) {
                const float4 a = *reinterpret_cast<const float4*>(p + 4 * i);
                f_[4 * i] = a.x; f_[4 * i + 1] = a.y; f_[4 * i + 2] = a.z; f_[4 * i + 3] = a.w;
            }
        }
    }
    __device__ __forceinline__ void to_f(float (&f)[N]) const {
#pragma unroll
        for (int i = 0; i < N; ++i) f[i] = f_[i];
    }
};

// A state row is split over L = 16 lanes (one DPP row, so its reductions need no cross-row
// step): dk / 16 values per lane.  Measured at 16/32 heads: at d = 128, rows over 32 lanes (4
// values each) ran 1.5x slower; at d = 64 and 32, rows over 8 and 4 lanes (8 values each)
// left most SIMDs without a wave and ran 1.8-1.9x slower.
template <int DK, int DV>
struct SeqShape {
    static constexpr int L = 16;                                   // lanes per row
    static constexpr int EPL = DK / L;                             // state values per lane
    static constexpr int NTH = DV * L < 256 ? DV * L : 256;       // threads per workgroup
    static constexpr int RPB = NTH / L;                            // rows per workgroup
    static constexpr int NBLK = DV / RPB;                          // workgroups per head
    static_assert((EPL == 2 || EPL == 4 || EPL == 8) && NBLK * RPB == DV, "sequential tiling");
};

// a . b over N values, as two interleaved FMA chains
template <int N>
__device__ __forceinline__ float dotn(const float (&a)[N], const float (&b)[N]) {
    float x = a[0] * b[0], y = a[1] * b[1];
#pragma unroll
    for (int e = 2; e < N; e += 2) {
        x = fmaf(a[e], b[e], x);
        y = fmaf(a[e + 1], b[e + 1], y);
    }
    return x + y;
}

template <typename E, int DK, int DV, bool NORM>
__global__ __launch_bounds__(256) void sequential_kernel(PrefillParams p) {
    using S = SeqShape<DK, DV>;
    using X = Elem<E>;
    constexpr int L = S::L, EPL = S::EPL;
    // tokens per prefetch block; lane `sub` of a row buffers the output of token `sub` of
    // the block, so a block is at most L tokens
    constexpr int U = (sizeof(E) == 2 ? 8 : 4) < L ? (sizeof(E) == 2 ? 8 : 4) : L;
    constexpr float LOG2E = 1.4426950408889634f;

    const int blk = blockIdx.x % S::NBLK;
    const int bh = blockIdx.x / S::NBLK;
    const int h = bh % p.Hv, b = bh / p.Hv;
    const int hk = h / (p.Hv / p.Hk);
    const int tid = threadIdx.x;
    const int sub = tid % L;
    const int i = blk * S::RPB + tid / L;   // state row (value index)
    const int T = p.T;

    // token t of this call is row (b * Ts + t0 + t) of the inputs; the per-token offsets
    // are uniform, the lane's own offset is added last
    const size_t tok0 = (size_t)b * p.Ts + p.t0;
    const E* kb = reinterpret_cast<const E*>(p.k) + (tok0 * p.Hk + hk) * DK;
    const E* qb = reinterpret_cast<const E*>(p.q) + (tok0 * p.Hk + hk) * DK;
    const E* vb = reinterpret_cast<const E*>(p.v) + (tok0 * p.Hv + h) * DV;
    const float* gb = p.g + tok0 * p.Hv + h;
    const float* bb = p.beta + tok0 * p.Hv + h;
    E* ob_base = reinterpret_cast<E*>(p.o) + (tok0 * p.Hv + h) * DV;
    const size_t rsk = (size_t)p.Hk * DK, rsv = (size_t)p.Hv * DV;
    const int koff = sub * EPL;

    struct Block {
        VecN<E, EPL> k[U], q[U];
        E v[U];
        float g[U], beta[U];
    };
    // tokens t0 .. t0 + U - 1 (indices past the end read the last token; never used)
    auto load = [&](Block& x, int t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = min(t0 + u, T - 1);
            x.k[u].load(kb + (size_t)t * rsk + koff);
            x.q[u].load(qb + (size_t)t * rsk + koff);
            x.v[u] = vb[(size_t)t * rsv + i];
            x.g[u] = gb[(size_t)t * p.Hv];
            x.beta[u] = bb[(size_t)t * p.Hv];
        }
    };

    float st[EPL];
    {
        const size_t srow = (((size_t)b * p.Hv + h) * DV + i) * DK + sub * EPL;
        VecN<float, EPL> s0;
        if (p.state_in) s0.load(p.state_in + srow);
        else
#pragma unroll
            for (int e = 0; e < EPL; ++e) s0.f_[e] = 0.f;
        s0.to_f(st);
    }

    // U tokens from a loaded block; GUARD: tokens past T are skipped (uniform branches)
    auto run = [&](const Block& x, int t0, auto guard) {
        constexpr bool GUARD = decltype(guard)::value;
        float ob = 0.f;   // output of token t0 + sub (lanes sub < U)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (GUARD && t0 + u >= T) break;
            float kk[EPL], qq[EPL];
            x.k[u].to_f(kk);
            x.q[u].to_f(qq);
            if constexpr (NORM) {   // the L lanes of a row hold the whole vector between them
                float ssk = dotn(kk, kk), ssq = dotn(qq, qq);
                group_sum2<L>(ssk, ssq);
                const float ik = rsqrtf(ssk + kNormEps), iq = rsqrtf(ssq + kNormEps);
#pragma unroll
                for (int e = 0; e < EPL; ++e) { kk[e] *= ik; qq[e] *= iq; }
            }
            const float a = __builtin_amdgcn_exp2f(x.g[u] * LOG2E);
            float kq = dotn(kk, qq), sk = dotn(st, kk), sq = dotn(st, qq);
            group_sum3<L>(sk, sq, kq);
            const float delta = x.beta[u] * (X::to_f(x.v[u]) - a * sk);
#pragma unroll
            for (int e = 0; e < EPL; ++e) st[e] = fmaf(delta, kk[e], a * st[e]);
            const float ou = fmaf(delta, kq, a * sq);
            ob = sub == u ? ou : ob;
        }
        if (sub < U && (!GUARD || t0 + sub < T)) ob_base[(size_t)(t0 + sub) * rsv + i] = X::from_f(ob);
    };

    // Two register sets, each loaded one block ahead of its use.  The main loop runs whole
    // pairs of blocks without bounds checks (straight-line code, so every wait is for the
    // set about to be used); the last 0 .. 2U - 1 tokens run guarded.
    Block A, Bk;
    load(A, 0);
    int t0 = 0;
    for (; t0 + 2 * U <= T; t0 += 2 * U) {
        load(Bk, t0 + U);
        run(A, t0, std::false_type{});
        load(A, t0 + 2 * U);
        run(Bk, t0 + U, std::false_type{});
    }
    if (t0 < T) {
        load(Bk, t0 + U);
        run(A, t0, std::true_type{});
        if (t0 + U < T) run(Bk, t0 + U, std::true_type{});
    }

    const size_t srow = (((size_t)b * p.Hv + h) * DV + i) * DK + sub * EPL;
    if constexpr (EPL == 2) {
        *reinterpret_cast<float2*>(p.state_out + srow) = make_float2(st[0], st[1]);
    } else {
#pragma unroll
        for (int e4 = 0; e4 < EPL; e4 += 4)
            *reinterpret_cast<float4*>(p.state_out + srow + e4) = make_float4(st[e4], st[e4 + 1], st[e4 + 2], st[e4 + 3]);
    }
}

template <typename E, int DK, int DV>
inline hipError_t launch_sequential(const PrefillParams& p, hipStream_t stream) {
    using S = SeqShape<DK, DV>;
    const dim3 grid((unsigned)(p.B * p.Hv * S::NBLK));
    if (p.qk_norm) return launch_kernel(sequential_kernel<E, DK, DV, true>, grid, dim3(S::NTH), stream, p);
    return launch_kernel(sequential_kernel<E, DK, DV, false>, grid, dim3(S::NTH), stream, p);
}

}  // namespace gdn
