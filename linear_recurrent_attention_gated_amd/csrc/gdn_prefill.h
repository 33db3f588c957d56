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
//   P[r,s] = exp(gamma_r - gamma_s) (q_r . k_s),  s <= r
//   U      = R diag(beta) (V - diag(Gamma) K S0^T)                  (deltas of the chunk)
//   O      = diag(Gamma) Q S0^T + P U
//   S_next = Gamma_{n-1} S0 + U^T diag(exp(gamma_{n-1} - gamma)) K
//
// Only exponentials of gamma_r - gamma_s with s <= r appear, so no factor can overflow.
// The state-independent factors are gathered around the residual Y = V - diag(Gamma) K S0^T
// (the values minus what the decayed state predicts for the chunk's keys):
//
//   Z   = K^T diag(exp(gamma_{n-1} - gamma)) R diag(beta)             (dk x n)
//   P'  = P R diag(beta)                                            (n x n, lower triangular)
//   S_next^T = Gamma_{n-1} S0^T + Z Y,      O = diag(Gamma) Q S0^T + P' Y
//
// so the scan reads v itself and nothing derived from it.
//
// Kernel 1 (intra_chunk_kernel), fully parallel over (batch, value head, chunk) items, run by
// a persistent grid that loads the next item while computing the current one: Gram blocks
// K K^T and K Q^T on MFMA, masks with the head's gates, (I + A) inverted in fp32 (16x16
// diagonal blocks by substitution, then block doubling on the fp32 matrix cores), Z and P' on
// MFMA.  Everything the scan needs goes to the workspace already arranged as MFMA operands
// (see "Workspace layout"), written straight from the accumulators.
//
// Kernel 2 (inter_chunk_kernel), one workgroup per (batch, value head, 16 state rows):
// rows of S evolve independently (each needs only its own entries of v), so a head's
// state is split into 16-row slices that never talk to each other.  The fp32 slice lives
// in MFMA accumulator registers for the whole scan and is written back once at the end
// ("Keep the recurrent state on chip": load the state once, carry it through the scan,
// write it after).  Each chunk's operands are fetched chunks ahead into registers, so the
// chunk-to-chunk chain waits only on LDS exchanges and matrix-core latency.
//
// Workspace layout (E = element type; a fragment is 64 lanes x KPL elements of a 16 x KB
// operand tile, lane l holding row l % 16).  Fragments marked "permuted" hold, in lane group
// g = l / 16, the k-values Elem<E>::kperm(kb, g, 0..KPL-1) of k-block kb; the others hold
// k = Elem<E>::doff(kb, g) + [0, KPL) (bf16: kb * KB + g * KPL; fp32: the permuted order as
// well).  The permuted order is the one an accumulator tile provides without lane exchanges
// (see gdn_device.h), and the scan reads the matching operand in the same order.  Fragment f
// of an array stands at Elem<E>::foff(f, lane): bf16 fragments one after another, fp32 ones in
// groups of four whose lane elements are adjacent, so every lane moves 16 bytes at a time.
//   KF  [B][Hk][N][C/16][DK/KB] fragments   A operand of K S^T   (rows tokens, k = dk) -- the raw k
//       rows (zero past the chunk's end), so the scan reads them contiguously
//   QF  [B][Hk][N][C/16][DK/KB] fragments   A operand of Q S^T   (rows tokens, k = dk) -- the raw q
//       rows, likewise
//   Z   [B][Hv][N][DK/16][NKC]  fragments   A operand of Z Y     (rows dk,     k = tokens; permuted)
//   P   [B][Hv][N][C/16][NKC]   fragments   A operand of P' Y    (rows tokens, k = tokens; permuted)
//   gam [B][Hv][N][2C + 4] fp32 gate factors per chunk: [0, C) the output scale exp(gamma_r),
//       [C, 2C) the key-row scale exp(gamma_r) of Y, [2C] the chunk decay exp(gamma_last)
//       (rows past the end repeat the last row's gamma).  With fused q/k normalisation the
//       output scale also carries 1 / |q_r| and the key-row scale 1 / |k_r|.
// NKC = ceil(C / KB); k-values past the chunk are stored as zeros.
#pragma once

#include <algorithm>
#include <atomic>
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
    void* KF;     // K row tiles as MFMA fragments, per key head (see the workspace layout)
    void* QF;     // Q row tiles as MFMA fragments, per key head
    void* Z;      // K^T diag(e) R diag(beta) as fragments, per value head
    void* P;      // P R diag(beta) as fragments, per value head
    float* gam;   // gate factors (see the workspace layout)
    int B, T, Hk, Hv, N;  // T = tokens of this pass, N = its number of chunks
    // Token t of batch b of this pass is token Ts * b + t0 + t of q, k, v, g, beta and o
    // (Ts = the arrays' tokens per batch, t0 = first token of the pass).  A prompt run in
    // several passes carries the state between them through state_out.
    int Ts, t0;
    // nonzero: q and k are L2-normalised per token and head inside the kernels
    int qk_norm;
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
    static constexpr size_t Z_PER_CHUNK = (size_t)(DK / 16) * NKC * FRAG;
    static constexpr int GATES = 2 * C + 4;   // fp32 gate factors per chunk (16-byte multiple)
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

// np (1, 2, 4 or 8; a compile-time constant after inlining) consecutive elements to dst, in
// the widest pieces its alignment (np * sizeof(E) bytes, or 16) allows
template <typename E>
__device__ __forceinline__ void store_run(E* dst, const E (&v)[8], int np) {
    const int bytes = np * (int)sizeof(E);
    if (bytes >= 16) {
        for (int o = 0; o < np; o += 16 / (int)sizeof(E)) {
            uint4 u;
            __builtin_memcpy(&u, v + o, 16);
            *reinterpret_cast<uint4*>(dst + o) = u;
        }
    } else if (bytes == 8) {
        uint2 u;
        __builtin_memcpy(&u, v, 8);
        *reinterpret_cast<uint2*>(dst) = u;
    } else if (bytes == 4) {
        uint32_t u;
        __builtin_memcpy(&u, v, 4);
        *reinterpret_cast<uint32_t*>(dst) = u;
    } else {
        dst[0] = v[0];
    }
}

// ------------------------------------------------------------------------------------
// Kernel 1: per-chunk, state-independent blocks; one work item per (batch, value head,
// chunk), four waves.
//
//   phase 0  the item's global loads, issued while the previous item is computed: K rows, g
//            and beta at the end of its phase 1; each wave's Q row tile as MFMA fragments and
//            one word of every 128-byte line of the chunk's v rows (see touch_v) as its phase 2
//            starts (fp32: ends)
//   phase 1  K rows and K^T (token-contiguous) into LDS; wave 0 scans the gates
//   phase 2  wave 0: Gram tiles of the diagonal blocks and of the first off-diagonal
//            level, masked into A; unit-lower-triangular 16x16 diagonal inverses by
//            substitution; first doubling level -- all wave-local.
//            every wave with a P row tile: that tile (K Q^T on MFMA, masked, kept as permuted
//            fragments) and, once per key head, its K and Q rows as fragments for the scan;
//            waves 1..3 also the remaining Gram tiles of A and zeros above the block diagonal.
//   phase 3  second doubling level (64-token chunks).  Every block of R is also written,
//            times beta and transposed, to a second LDS array that phase 4 reads
//   phase 4  Z^T = diag(beta) R^T diag(e) K and P'^T = diag(beta) R^T P^T on MFMA, stored from
//            the accumulators as permuted fragments of Z and P'
// A is overwritten in place by R = (I + A)^-1.
// ------------------------------------------------------------------------------------

// 2^x with the hardware instruction (results below the fp32 normal range flush to zero,
// which is what the decay factors that use it need)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// wave-local ordering point for LDS traffic exchanged between lanes of one wave
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// NORM: q and k are L2-normalised (p.qk_norm); a separate instantiation, so that the plain
// path carries none of its registers.
template <typename E, int DK, int DV, int C, bool NORM>
// Two workgroups per CU in both builds: the fp32 one (69 KB of LDS without the K^T copy) then
// spills a few registers, and still runs ~25% faster than with one workgroup per CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void intra_chunk_kernel(PrefillParams p) {
    using S = PrefillShape<E, DK, DV, C>;
    using X = Elem<E>;
    typedef typename X::frag frag;
    constexpr int KB = S::KB, KPL = S::KPL, NT = S::NT, NKD = S::NKD, NKC = S::NKC;
    constexpr int EPV = 16 / (int)sizeof(E);   // elements per 16-byte vector
    constexpr int LDK = DK + EPV;              // K rows
    constexpr int CP = NKC * KB;               // chunk width padded to whole k-blocks
    constexpr int LDT = CP + EPV;              // token-contiguous rows (K^T)
    constexpr int LDR = CP + 4;                // fp32 A / R rows
    constexpr int ND = DK / 16;
    static_assert(NT == 1 || NT == 2 || NT == 4, "chunk of 16, 32 or 64 tokens");
    constexpr float LOG2E = 1.4426950408889634f;
    // a k-block of an operand fragment spans the tokens [kb_lo(kb), kb_lo(kb) + KSPAN) (bf16:
    // 32 consecutive tokens; fp32: four tokens of one 16-token tile, see Elem::kperm)
    constexpr int KSPAN = KB > 16 ? KB : 16;
    auto kb_lo = [](int kb) { return kb * KB / KSPAN * KSPAN; };

    __shared__ __align__(16) E Ks[C * LDK];
    // token-contiguous K^T rows: the B operand of phase 4 needs 8 consecutive tokens of one dk
    // column per lane in bf16; an fp32 fragment is one element per lane, read from Ks directly
    constexpr bool TRK = KPL == 8;
    __shared__ __align__(16) E KsT[TRK ? DK * LDT : 4];
    __shared__ __align__(16) float sR[C * LDR];    // A, then R in place
    __shared__ __align__(16) float sRT[C * LDR];   // row s: beta_s R[r][s] for r < CP (zero past C)
    __shared__ __align__(16) float sg2[C];         // gamma * log2(e)
    __shared__ __align__(16) float sbeta[CP];
    __shared__ __align__(16) float se[CP];         // update scale exp(gamma_last - gamma_r)
    // fused normalisation (NORM only): |k_r|^2 in parts, one per 16-byte column block of the
    // rows (written where the rows are stored to LDS), and 1 / |k_r| formed from them by every
    // wave into its own copy, so that no barrier is spent on it
    constexpr int VKN = DK / EPV;   // column blocks of a K row
    __shared__ __align__(16) float sk2p[NORM ? C * (VKN + 1) : 4];
    __shared__ __align__(16) float sinvk[NORM ? 4 * CP : 4];

    const int T = p.T, Hk = p.Hk, Hv = p.Hv, N = p.N;
    const int grp = Hv / Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rl = lane & 15, g = lane >> 4, kq = g * KPL, rq = g * 4;
    const size_t rsk = (size_t)Hk * DK, rsv = (size_t)Hv * DV;
    const float* winvk = sinvk + (NORM ? wave * CP : 0);
    auto invk = [&](int r) { return NORM ? winvk[r] : 1.f; };
    auto invk4 = [&](int r) {
        if constexpr (NORM) return *reinterpret_cast<const float4*>(winvk + r);
        return make_float4(1.f, 1.f, 1.f, 1.f);
    };
    float invq = 1.f;   // 1 / |q_r| of this lane's row of the wave's P row tile (NORM)

    // Work items are (batch, chunk, value head).  Item i takes value head (i / 8) % grp of
    // "rest" (i / (8 grp)) * 8 + i % 8, which names (batch, chunk, key head): with a grid that
    // is a multiple of 8 grp, the value heads sharing a key head run at the same time on one
    // XCD (items i and i + 8 go to workgroups 8 apart), so their K and Q rows are read once
    // into that XCD's L2.
    const int nrest = p.B * N * Hk;
    const int nitems = (nrest + 7) / 8 * 8 * grp;
    auto rest_of = [&](int i) { return (i / (8 * grp)) * 8 + i % 8; };
    auto valid = [&](int i) { return i < nitems && rest_of(i) < nrest; };
    struct Item { int b, c, h; };
    auto decode = [&](int i) {
        const int r = rest_of(i);
        Item it;
        it.b = r / (N * Hk);
        it.c = (r / Hk) % N;
        it.h = (r % Hk) * grp + (i / 8) % grp;
        return it;
    };

    // ---- loads of an item (rows past the chunk's end read row n - 1 and are zeroed later) ----
    constexpr int VK = DK / EPV;
    constexpr int PK = (C * VK + kThreads - 1) / kThreads;
    // v: this kernel does not use it, but the scan reads it on its critical path in 32-byte
    // pieces per row and state slice.  One 4-byte read of each 128-byte line of the chunk's v
    // rows here (by waves 1..3, after the next item's Q loads) brings them into the last-level
    // cache while they are off that path; the words read are folded into vsink, which only an
    // impossible condition stores.
    constexpr int LPR = (DV * (int)sizeof(E) + 127) / 128;   // lines per v row
    constexpr int NVL = (C * LPR + kThreads - 65) / (kThreads - 64);
    // this wave's P row tile: wave 0 takes row 0, wave w >= 1 row NT - w (if >= 1)
    const int pm = wave == 0 ? 0 : NT - wave;
    const bool has_prow = wave == 0 || pm >= 1;
    const int pm_ld = max(pm, 0);
    uint4 kr[PK];
    uint32_t vl[NVL] = {};
    uint32_t vsink = 0;
    frag qf[NKD];
    // bf16: the next item's Q fragments arrive in registers of their own, loaded as phase 2
    // starts; fp32 (twice the registers) reloads qf once phase 2 is done with it
    constexpr bool QN = KPL == 8;
    frag qn[QN ? NKD : 1];
    float graw, braw;
    auto load_kg = [&](const Item& it) {
        const int t0 = it.c * C, n = min(C, T - t0);
        const E* kg = reinterpret_cast<const E*>(p.k) + ((size_t)it.b * p.Ts + p.t0 + t0) * rsk + (size_t)(it.h / grp) * DK;
        // thread tid holds vectors tid * PK + [0, PK): PK consecutive tokens of one column block
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int idx = min(tid * PK + i, C * VK - 1), r = idx % C, cv = idx / C;
            kr[i] = *reinterpret_cast<const uint4*>(kg + (size_t)min(r, n - 1) * rsk + cv * EPV);
        }
        // the gates go to wave 0 alone, which scans them (a token's gates of all heads share a
        // 128-byte line, so each of these loads touches 64 lines)
        if (wave == 0) {
            const size_t gidx = ((size_t)it.b * p.Ts + p.t0 + t0 + min(lane, n - 1)) * Hv + it.h;
            graw = p.g[gidx];
            braw = p.beta[gidx];
        }
    };
    auto touch_v = [&](const Item& it) {   // waves 1..3
        const int t0 = it.c * C, n = min(C, T - t0);
        const E* vg = reinterpret_cast<const E*>(p.v) + ((size_t)it.b * p.Ts + p.t0 + t0) * rsv + (size_t)it.h * DV;
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int idx = min(tid - 64 + i * (kThreads - 64), C * LPR - 1), r = idx / LPR, ln = idx % LPR;
            vl[i] = *reinterpret_cast<const uint32_t*>(vg + (size_t)min(r, n - 1) * rsv + ln * (128 / (int)sizeof(E)));
        }
    };
    auto load_q = [&](const Item& it, frag (&dst)[NKD]) {
        const int t0 = it.c * C, n = min(C, T - t0);
        const E* qg = reinterpret_cast<const E*>(p.q) + ((size_t)it.b * p.Ts + p.t0 + t0) * rsk + (size_t)(it.h / grp) * DK;
        const E* src = qg + (size_t)min(pm_ld * 16 + rl, n - 1) * rsk;
#pragma unroll
        for (int kb = 0; kb < NKD; kb += X::GRP) X::ld_grp(src + X::doff(kb, g), &dst[kb]);
    };

    int item = blockIdx.x;
    if (!valid(item)) return;
    Item cur = decode(item);
    load_kg(cur);
    load_q(cur, qf);
    if (wave > 0) touch_v(cur);
    for (;;) {
    const int c = cur.c, h = cur.h, b = cur.b;
    const int hk = h / grp;
    const int t0 = c * C;
    const int n = min(C, T - t0);
    const size_t bh = (size_t)b * Hv + h;
    // the next item's loads are issued while this one is computed
    const int next = item + (int)gridDim.x;
    const bool more = valid(next);
    const Item nxt = decode(more ? next : item);

    // ---- phase 1: K rows and K^T into LDS; gates -----------------------------------------------
    // The item's prefetched registers are opaque until here, so that nothing derived from them
    // is computed (and waited for) right after their loads were issued, an item earlier.
#pragma unroll
    for (int i = 0; i < PK; ++i) reg_fence(kr[i]);
    // rows to Ks; the transpose takes each thread's PK consecutive tokens of a column as one
    // contiguous run per column
    if (tid * PK < C * VK) {
        const int r0 = (tid * PK) % C, cv = (tid * PK) / C;
        E el[PK][EPV];
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const uint4 z = {0u, 0u, 0u, 0u};
            const uint4 a = r0 + i < n ? kr[i] : z;
            *reinterpret_cast<uint4*>(Ks + (r0 + i) * LDK + cv * EPV) = a;
            const E* e = reinterpret_cast<const E*>(&a);
#pragma unroll
            for (int j = 0; j < EPV; ++j) el[i][j] = e[j];
            if constexpr (NORM) {
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < EPV; ++j) {
                    const float x = X::to_f(e[j]);
                    ss += x * x;
                }
                sk2p[(r0 + i) * (VKN + 1) + cv] = ss;
            }
        }
        if constexpr (TRK) {
#pragma unroll
            for (int j = 0; j < EPV; ++j) {
                E run[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) run[i] = el[i < PK ? i : 0][j];
                store_run(KsT + (cv * EPV + j) * LDT + r0, run, PK);
            }
        }
    }
    if (TRK && CP > C) {   // token columns past the chunk (16-token chunks in bf16)
        for (int e = tid; e < DK * (CP - C); e += kThreads) {
            const int d = e / (CP - C), s = C + e % (CP - C);
            KsT[d * LDT + s] = X::from_f(0.f);
        }
    }
    if (wave == 0) {
        // running log-gate; constant past the end
        const float x = wave_prefix_sum(lane < n ? graw : 0.f);
        const float bt = lane < n ? braw : 0.f;
        const float x2 = x * LOG2E;
        const float gl2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x2), C - 1));
        if (lane < C) sg2[lane] = x2;
        if (lane < CP) {
            sbeta[lane] = bt;
            se[lane] = lane < C ? exp2f(gl2 - x2) : 0.f;   // with NORM: divided by |k_r| in phase 2
        }
        if constexpr (!NORM) {   // gate factors for the scan (with NORM: in phase 2, scaled)
            float* gf = p.gam + (bh * N + c) * S::GATES;
            if (lane < C) {
                gf[lane] = exp2f(x2);
                gf[C + lane] = exp2f(x2);
            }
            if (lane == 0) gf[2 * C] = exp2f(gl2);
        }
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) vsink ^= vl[i];
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) qf[kb] = X::keep_if(qf[kb], pm_ld * 16 + rl < n);
    // every register loaded for this item is taken before the next item's loads are issued:
    // the count of outstanding loads drains in issue order, so a wait for one of them placed
    // after those loads would wait for them too
#pragma unroll
    for (int kb = 0; kb < NKD; ++kb) reg_fence(qf[kb]);
    reg_fence(vsink);
    asm volatile("" ::: "memory");
    if (more) load_kg(nxt);   // registers consumed above; the next item's rows are in flight from here
    lds_barrier();   // (B1)
    if constexpr (NORM) {
        // 1 / |k_r| into this wave's copy (lane r sums row r's parts; rows past the chunk are
        // zero), 1 / |q_r| from the wave's Q row tile (lane groups hold a quarter of a row each)
        float* w = sinvk + wave * CP;
        if (lane < C) {
            float ss = 0.f;
#pragma unroll
            for (int v = 0; v < VKN; ++v) ss += sk2p[lane * (VKN + 1) + v];
            w[lane] = rsqrtf(ss + kNormEps);
        } else if (lane < CP) {
            w[lane] = 1.f;
        }
        if (has_prow) {
            float ss = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb)
#pragma unroll
                for (int e = 0; e < KPL; ++e) {
                    const float x = X::to_f(frag_elem(qf[kb], e));
                    ss += x * x;
                }
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            invq = rsqrtf(ss + kNormEps);
        }
        wave_lds_sync();
    }
    // with NORM, the gate factors of this wave's P rows, scaled by the norms (before the end of
    // phase 2: phase 4 reads se)
    auto norm_gates = [&] {
        if constexpr (NORM) {
            float* gf = p.gam + (bh * N + c) * S::GATES;
            if (has_prow && g == 0) {
                const int r = pm * 16 + rl;
                const float gr = exp2f(sg2[r]), ik = invk(r);
                gf[r] = gr * invq;
                gf[C + r] = gr * ik;
                se[r] *= ik;
            }
            if (wave == 0 && lane == 0) gf[2 * C] = exp2f(sg2[C - 1]);
        }
    };

    // Gram tile of K rows: D[r][s] = k_r . k_s  (r in tile tm, s in tile tn)
    auto kk_tile = [&](int tm, int tn) {
        const E* ar = Ks + (tm * 16 + rl) * LDK;
        const E* br = Ks + (tn * 16 + rl) * LDK;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < NKD; kb += X::GRP) {
            frag a[X::GRP], bb[X::GRP];
            X::ld_grp(ar + X::doff(kb, g), a);
            X::ld_grp(br + X::doff(kb, g), bb);
#pragma unroll
            for (int i = 0; i < X::GRP; ++i) acc = X::mma(a[i], bb[i], acc);
        }
        return acc;
    };
    // A[r][s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s) for s < r, from a Gram tile
    auto mask_a = [&](int tm, int tn, f32x4 G) {
        const int s = tn * 16 + rl;
        const float gs = sg2[s], ks = invk(s);
        const float4 gr = *reinterpret_cast<const float4*>(sg2 + tm * 16 + rq);
        const float4 br = *reinterpret_cast<const float4*>(sbeta + tm * 16 + rq);
        const float4 kr4 = invk4(tm * 16 + rq);
        const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, brv[4] = {br.x * kr4.x, br.y * kr4.y, br.z * kr4.z, br.w * kr4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = tm * 16 + rq + j;
            sR[r * LDR + s] = (s < r) ? brv[j] * ks * fast_exp2(grv[j] - gs) * G[j] : 0.f;
        }
    };
    // P row tile m: P[r][s] = exp(gamma_r - gamma_s) (q_r . k_s), s <= r, as permuted A-operand
    // fragments (rows r, k = s) built from tiles D[s][r] = K_t Q_m^T; kept for phase 4
    frag pk[NKC];
    auto p_row = [&](int m) {
        const int r = m * 16 + rl;
        const float gr = sg2[r], qs = invq;   // (this wave's own row tile)
        auto ptile = [&](int t) {
            f32x4 acc = zero4();
            if (t <= m) {
                const E* ar = Ks + (t * 16 + rl) * LDK;
#pragma unroll
                for (int kb = 0; kb < NKD; kb += X::GRP) {
                    frag a[X::GRP];
                    X::ld_grp(ar + X::doff(kb, g), a);
#pragma unroll
                    for (int i = 0; i < X::GRP; ++i) acc = X::mma(a[i], qf[kb + i], acc);
                }
                const float4 gs = *reinterpret_cast<const float4*>(sg2 + t * 16 + rq);
                const float4 ks = invk4(t * 16 + rq);
                const float gsv[4] = {gs.x, gs.y, gs.z, gs.w}, ksv[4] = {ks.x, ks.y, ks.z, ks.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = t * 16 + rq + j;
                    acc[j] = (s <= r) ? qs * ksv[j] * fast_exp2(gr - gsv[j]) * acc[j] : 0.f;
                }
            }
            return acc;
        };
        if constexpr (KPL == 8) {
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                pk[kb] = 2 * kb <= m ? X::pack(ptile(2 * kb), 2 * kb + 1 < NT ? ptile(2 * kb + 1) : zero4()) : X::zero();
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 d = ptile(t);
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[4 * t + j] = d[j];
            }
        }
    };

    // this wave's K and Q row tiles m as fragments for the scan's products with the state,
    // once per key head (rows past the chunk are zero)
    auto store_rows = [&](int m) {
        if (h % grp != 0) return;
        const size_t off = (((size_t)b * Hk + hk) * N + c) * S::W_PER_CHUNK;
        E* KFg = reinterpret_cast<E*>(p.KF) + off;
        E* QFg = reinterpret_cast<E*>(p.QF) + off;
        const E* krow = Ks + (m * 16 + rl) * LDK;
        const size_t tile = (size_t)m * NKD * 64 * KPL;   // (NKD is a multiple of the group)
#pragma unroll
        for (int kb = 0; kb < NKD; kb += X::GRP) {
            const size_t f = tile + X::foff(kb, lane);
            *reinterpret_cast<uint4*>(KFg + f) = *reinterpret_cast<const uint4*>(krow + X::doff(kb, g));
            X::st_grp(QFg + f, &qf[kb]);
        }
    };

    // ---- phase 2 -------------------------------------------------------------------------------
    // bf16: the next item's Q rows and v lines, a whole item ahead of their use, in code common
    // to all waves (see below for why not inside the branches)
    if constexpr (QN) {
        if (more) {
            load_q(nxt, qn);
            if (wave > 0) touch_v(nxt);
        }
    }
    if (wave == 0) {
        f32x4 Gd[NT];
#pragma unroll
        for (int d = 0; d < NT; ++d) Gd[d] = kk_tile(d, d);
        p_row(0);
        store_rows(0);
#pragma unroll
        for (int d = 0; d < NT; ++d) mask_a(d, d, Gd[d]);
        wave_lds_sync();
        // (I + A_dd)^-1 of each 16x16 diagonal block by forward substitution: lane (d, j)
        // computes column j of block d
        if (g < NT) {
            float* Ab = sR + (g * 16) * LDR + g * 16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float a[16];
#pragma unroll
                for (int m4 = 0; m4 < (r + 3) / 4; ++m4) {
                    const float4 v = *reinterpret_cast<const float4*>(Ab + r * LDR + 4 * m4);
                    a[4 * m4] = v.x; a[4 * m4 + 1] = v.y; a[4 * m4 + 2] = v.z; a[4 * m4 + 3] = v.w;
                }
                float s0 = (r == rl) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) {
                    if (m & 1) s1 -= a[m] * x[m];
                    else s0 -= a[m] * x[m];
                }
                x[r] = s0 + s1;
            }
            wave_lds_sync();
#pragma unroll
            for (int r = 0; r < 16; ++r) Ab[r * LDR + rl] = x[r];
            // the same column, times beta, as a row of (R diag(beta))^T
            float* At = sRT + (g * 16 + rl) * LDR + g * 16;
            const float bs = sbeta[g * 16 + rl];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<float4*>(At + 4 * r4) =
                    make_float4(bs * x[4 * r4], bs * x[4 * r4 + 1], bs * x[4 * r4 + 2], bs * x[4 * r4 + 3]);
        }
    } else {
        if (has_prow) {
            p_row(pm);
            store_rows(pm);
        }
        // the A21 tiles of the 32x32 diagonal blocks (2q + 1, 2q): q = 0 on wave 1, q = 1 on wave 3
        if ((NT >= 2 && wave == 1) || (NT == 4 && wave == 3)) {
            const int q = wave >> 1;
            mask_a(2 * q + 1, 2 * q, kk_tile(2 * q + 1, 2 * q));
        }
        if (NT == 4 && wave >= 2) {   // the 32x32 off-diagonal block, one tile column per wave
            const int tn = wave - 2;
            const f32x4 Ga = kk_tile(2, tn), Gb = kk_tile(3, tn);
            mask_a(2, tn, Ga);
            mask_a(3, tn, Gb);
        }
        // the zeros of (R diag(beta))^T: row s, tokens r of earlier 16-token blocks (R is lower
        // triangular) and past the chunk (phase 4 reads whole rows)
        constexpr int CV = CP / 4;
        for (int e = tid - 64; e < C * CV; e += kThreads - 64) {
            const int s = e / CV, r4 = (e % CV) * 4;
            if ((r4 >> 4) < (s >> 4) || r4 >= C)
                *reinterpret_cast<float4*>(sRT + s * LDR + r4) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    if constexpr (NT >= 2) {
        lds_barrier();   // (B2a) diagonal blocks inverted, A21 tiles masked
        // first doubling level, R21 = -R22 (A21 R11), one block pair (2q, 2q + 1) per wave 2 + q
        if (wave >= 2 && wave - 2 < NT / 2) {
            const int q = wave - 2;
            const int lo = 32 * q, hi = lo + 16;
            // k runs in the order 4 g + kb (as in the accumulator tiles), so that a lane's four
            // A values are one 16-byte run and the B reads of a k-step fall on distinct banks
            f32x4 t = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                t = mma4(sR[(hi + rl) * LDR + lo + 4 * g + kb], sR[(lo + 4 * g + kb) * LDR + lo + rl], t);
            f32x4 r21 = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) r21 = mma4(sR[(hi + rl) * LDR + hi + 4 * g + kb], t[kb], r21);
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < 4; ++j) sR[(hi + rq + j) * LDR + lo + rl] = -r21[j];
            const float bs = -sbeta[lo + rl];
            *reinterpret_cast<float4*>(sRT + (lo + rl) * LDR + hi + rq) =
                make_float4(bs * r21[0], bs * r21[1], bs * r21[2], bs * r21[3]);
        }
    }
    // fp32: the next item's Q rows (and v lines) are loaded here, after the branches of phase 2
    // rather than inside them: a register loaded in one branch and reused in the other would
    // otherwise be waited for in both, and the branch of wave 0 would wait for the next item's
    // K rows.
    if (!QN && more) {
        load_q(nxt, qf);
        if (wave > 0) touch_v(nxt);
    }
    norm_gates();
    lds_barrier();   // (B2)

    // ---- phase 3: second doubling level (32x32 blocks) -----------------------------------------
    // Only (R diag(beta))^T is read after this level, so its block R21 goes there alone.
    if constexpr (NT == 4) {
        if (wave < 2) {
            const int tj = wave;   // tile column of T and R21
            // T = A21 R11 (32 x 32, column tile tj); R11 is zero above its diagonal; k in the
            // order 16 blk + 4 g + kb, as in the first level
            f32x4 t0v = zero4(), t1v = zero4();
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                if (blk >= tj) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const int k = 16 * blk + 4 * g + kb;
                        const float bv = sR[k * LDR + tj * 16 + rl];
                        t0v = mma4(sR[(32 + rl) * LDR + k], bv, t0v);
                        t1v = mma4(sR[(48 + rl) * LDR + k], bv, t1v);
                    }
                }
            }
            // R21 = -R22 T; R22 rows 32..47 see T rows 0..15, rows 48..63 all of T
            f32x4 u0 = zero4(), u1 = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                u0 = mma4(sR[(32 + rl) * LDR + 32 + 4 * g + kb], t0v[kb], u0);
                u1 = mma4(sR[(48 + rl) * LDR + 32 + 4 * g + kb], t0v[kb], u1);
                u1 = mma4(sR[(48 + rl) * LDR + 48 + 4 * g + kb], t1v[kb], u1);
            }
            const float bs = -sbeta[tj * 16 + rl];
            float* At = sRT + (tj * 16 + rl) * LDR;
            *reinterpret_cast<float4*>(At + 32 + rq) = make_float4(bs * u0[0], bs * u0[1], bs * u0[2], bs * u0[3]);
            *reinterpret_cast<float4*>(At + 48 + rq) = make_float4(bs * u1[0], bs * u1[1], bs * u1[2], bs * u1[3]);
        }
        lds_barrier();   // (B3) R complete
    }

    // ---- phase 4: Z and P' ------------------------------------------------------------------
    // Both are stored as permuted A-operand fragments, so each is formed transposed: an
    // accumulator tile with columns = the operand's rows.  A operands come from rows of sRT.
    {
        // Z^T tile (s-tile u, dk-tile dt) = sum over tokens r of (beta_s R[r][s] e_r) K[r][d].
        E* Zg = reinterpret_cast<E*>(p.Z) + (bh * N + c) * S::Z_PER_CHUNK;
        if constexpr (KPL == 1 && NT == 4 && ND == 8) {
            // fp32, 64-token chunks, dk = 128: s-tile u needs the k-blocks from 4u on (16 - 4u
            // products per dk tile), so wave w takes s-tile w for dk tiles 0..3 and s-tile 3 - w
            // for 4..7 (the same count for every wave), two dk tiles at a time as independent
            // product chains
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int u = half == 0 ? wave : NT - 1 - wave;
                const float* row = sRT + (u * 16 + rl) * LDR;
                frag a[NKC];
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) a[kb] = kb >= 4 * u ? row[kb * KB + kq] * se[kb * KB + kq] : 0.f;
#pragma unroll
                for (int d2 = 0; d2 < 4; d2 += 2) {
                    const int dt = half * 4 + d2;
                    f32x4 c0 = zero4(), c1 = zero4();
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb) {
                        if (kb >= 4 * u) {
                            const E* kc = Ks + (kb * KB + kq) * LDK + dt * 16 + rl;
                            c0 = X::mma(a[kb], kc[0], c0);
                            c1 = X::mma(a[kb], kc[16], c1);
                        }
                    }
                    const frag f0[4] = {c0[0], c0[1], c0[2], c0[3]}, f1[4] = {c1[0], c1[1], c1[2], c1[3]};
                    X::st_grp(Zg + (size_t)dt * NKC * 64 * KPL + X::foff(4 * u, lane), f0);
                    X::st_grp(Zg + (size_t)(dt + 1) * NKC * 64 * KPL + X::foff(4 * u, lane), f1);
                }
            }
        } else {
            // The waves split Z's stored k-blocks: a group is the TPG s-tiles one k-block of Z holds.
            constexpr int TPG = KPL == 8 ? 2 : 1;
            constexpr int NG = (NT + TPG - 1) / TPG;
            const int zg = wave % NG;
            frag az[TPG][NKC];
#pragma unroll
            for (int i = 0; i < TPG; ++i) {
                const int u = zg * TPG + i;
                const float* row = sRT + (min(u, NT - 1) * 16 + rl) * LDR;   // (s-tiles past the chunk: unused)
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    az[i][kb] = X::zero();
                    if (u < NT && kb_lo(kb) + KSPAN > u * 16) {   // blocks wholly before s-tile u are zero
                        float t[KPL];
#pragma unroll
                        for (int e = 0; e < KPL; ++e) t[e] = row[kb * KB + kq + e] * se[kb * KB + kq + e];
                        az[i][kb] = X::ld_f(t);
                    }
                }
            }
            for (int dt = wave / NG; dt < ND; dt += 4 / NG) {
                // B operand: K^T rows (dk) over tokens -- from KsT (bf16) or a column of Ks (fp32)
                auto kt = [&](int kb) {
                    if constexpr (TRK) return X::ld(KsT + (dt * 16 + rl) * LDT + kq + kb * KB);
                    else return X::ld(Ks + (kb * KB + kq) * LDK + dt * 16 + rl);
                };
                f32x4 acc[TPG];
#pragma unroll
                for (int i = 0; i < TPG; ++i) acc[i] = zero4();
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    const frag bk = kt(kb);
#pragma unroll
                    for (int i = 0; i < TPG; ++i) {
                        const int u = zg * TPG + i;
                        if (u < NT && kb_lo(kb) + KSPAN > u * 16) acc[i] = X::mma(az[i][kb], bk, acc[i]);
                    }
                }
                if constexpr (KPL == 8) {
                    *reinterpret_cast<frag*>(Zg + ((size_t)(dt * NKC + zg) * 64 + lane) * KPL) = X::pack(acc[0], acc[TPG - 1]);
                } else {   // fragments 4 zg .. 4 zg + 3: one lane group
                    const frag f[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
                    X::st_grp(Zg + (size_t)dt * NKC * 64 * KPL + X::foff(4 * zg, lane), f);
                }
            }
        }

        // P'^T tile (s-tile u, row tile m) = sum over tokens t of beta_s R[t][s] P[r][t]: the
        // P fragments kept from phase 2 are the B operand (k = t in the permuted order)
        if (has_prow) {
            const int m = pm;
            f32x4 acc[NT];
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                acc[u] = zero4();
                if (u > m) continue;
                const float* row = sRT + (u * 16 + rl) * LDR;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    if (kb_lo(kb) > m * 16 + 15 || kb_lo(kb) + KSPAN <= u * 16) continue;
                    float t[KPL];
#pragma unroll
                    for (int e = 0; e < KPL; ++e) t[e] = row[X::kperm(kb, g, e)];
                    acc[u] = X::mma(X::ld_f(t), pk[kb], acc[u]);
                }
            }
            // fragments wholly above the diagonal (tokens past row tile m) are never written:
            // the scan does not read them
            E* Pg = reinterpret_cast<E*>(p.P) + (bh * N + c) * S::P_PER_CHUNK;
            if constexpr (KPL == 8) {
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    if (2 * kb > m) break;
                    *reinterpret_cast<frag*>(Pg + ((size_t)(m * NKC + kb) * 64 + lane) * KPL) =
                        X::pack(acc[2 * kb], 2 * kb + 1 < NT ? acc[2 * kb + 1] : zero4());
                }
            } else {
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    if (u > m) break;
                    const frag f[4] = {acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
                    X::st_grp(Pg + (size_t)m * NKC * 64 * KPL + X::foff(4 * u, lane), f);
                }
            }
        }
    }
    if (!more) break;
    if constexpr (QN) {
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) qf[kb] = qn[kb];
    }
    lds_barrier();   // this item's LDS reads are done before the next item overwrites it
    item = next;
    cur = nxt;
    }
    // keeps the v reads above (the value cannot match and T is never negative)
    if (vsink == 0x9E3779B9u && T < 0) p.gam[0] = 0.f;
}

// ------------------------------------------------------------------------------------
// Kernel 2: chunks in order; fp32 state slice in accumulator registers.
//
// Eight waves per workgroup in two roles.  Chain waves 0..3 carry the recurrence: the
// residual Y = V - diag(Gamma) K S^T for their 16-token tile, then S^T <- Gamma_n S^T + Z Y for
// their state tiles.  Output waves 4..7 compute O = Gamma (Q S^T) + P' Y for their token tile
// one barrier behind, from a double-buffered copy of the state, so the output products stay
// off the chain.  Both roles form their token tiles transposed (state rows by tokens), so that
// each lane holds four consecutive state rows of one token: 8 contiguous bytes of v to read or
// of o to write (16 in fp32).  Each role prefetches its own
// operands NB chunks ahead into registers; the chain waves issue those loads just before the
// barriers they would wait at anyway, not between a barrier and the next chunk's products.
// SPLIT: feed the state to K S^T as a bf16 hi + lo pair (two MFMAs) so the residual Y sees
// the fp32 state to ~16 bits instead of 8.
// ------------------------------------------------------------------------------------
constexpr int kScanThreads = 512;
// operand sets in flight per wave: chain waves are on the critical path and prefetch
// deeper; fp32 operands take four times the registers of bf16 ones
template <typename E> struct ScanDepth;
// (v, read from the caller's array rather than the workspace, is held in sets of its own:
// vrows, a multiple of chain; fetching it 6 chunks ahead instead of 3 measured no faster)
template <> struct ScanDepth<bf16_t> { static constexpr int chain = 3, output = 2, vrows = 3; };
template <> struct ScanDepth<float> { static constexpr int chain = 2, output = 1, vrows = 2; };

template <typename E, int DK, int C, int TPW>
struct ChainOperands {
    using X = Elem<E>;
    typedef typename X::frag frag;
    static constexpr int NKD = DK / X::KB;
    static constexpr int NKC = (C + X::KB - 1) / X::KB;
    frag kf[NKD];       // K row tile (rows tokens, k = dk)
    frag z[TPW][NKC];   // Z rows of this wave's state tiles (rows dk, k = tokens; permuted)
    float gk;           // key-row scale of this lane's token row
    float gn;           // chunk decay exp(gamma_last)
};

template <typename E, int DK, int C>
struct OutputOperands {
    using X = Elem<E>;
    typedef typename X::frag frag;
    static constexpr int NKD = DK / X::KB;
    static constexpr int NKC = (C + X::KB - 1) / X::KB;
    frag q[NKD];
    frag p[NKC];
    float gr;     // output scale of this lane's token
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
    constexpr int NBC = ScanDepth<E>::chain, NBO = ScanDepth<E>::output, NBV = ScanDepth<E>::vrows;
    static_assert(NBV % NBC == 0, "v sets cycle with the operand sets");
    typedef ChainOperands<E, DK, C, TPW> COps;
    typedef OutputOperands<E, DK, C> OOps;

    __shared__ __align__(16) E Sb[2][16 * LDS_];              // state slice, hi part, 2 buffers
    __shared__ __align__(16) E Sl[2][SPLIT ? 16 * LDS_ : EPV];  // lo part
    __shared__ __align__(16) E YT[16 * LDU];                   // Y^T (for Z Y and P' Y)

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
    const int rl = lane & 15, g = lane >> 4, rq = g * 4;
    const bool chain = wave < 4;
    const int w4 = wave & 3;
    const bool has_tile = w4 < NT;
    const int m = w4 % NT;           // token tile (duplicate for waves past the chunk's tiles)
    const int Nf = T / C;            // full chunks; a partial last chunk takes the tail path
    std::integral_constant<bool, false> full;
    std::integral_constant<bool, true> tail;

    const float* gates = p.gam + (size_t)bh * N * Sh::GATES;   // per chunk: see the workspace layout

    for (int e = tid; e < 16 * LDU; e += kScanThreads) {   // columns past the chunk read as zero
        YT[e] = X::from_f(0.f);
    }

    if (chain) {
        // the chain is the critical path: its waves win instruction arbitration on their SIMDs
        __builtin_amdgcn_s_setprio(3);
        const E* KFg = reinterpret_cast<const E*>(p.KF) + ((size_t)b * Hk + hk) * N * Sh::W_PER_CHUNK
                       + (size_t)m * NKD * Sh::FRAG;
        const E* Zg = reinterpret_cast<const E*>(p.Z) + (size_t)bh * N * Sh::Z_PER_CHUNK;
        // v of this lane's token row (rl) of tile m, state rows i0 + rq + [0, 4)
        const E* vg = reinterpret_cast<const E*>(p.v) + (size_t)h * DV + i0 + rq;

        // a later chunk's operands are fetched in parts, each issued where its registers are
        // free and this wave would otherwise wait: K rows and the key-row scales once Y is
        // formed (before the first barrier), v (NBV chunks ahead) right after that barrier, Z
        // and the decay once the update has read them (before the second)
        auto fetch_w = [&](COps& op, int c) {
            const float* gc = gates + (size_t)c * Sh::GATES;
            op.gk = gc[C + m * 16 + rl];
            const E* ksrc = KFg + (size_t)c * Sh::W_PER_CHUNK;
#pragma unroll
            for (int kb = 0; kb < NKD; kb += X::GRP) X::ld_grp(ksrc + X::foff(kb, lane), &op.kf[kb]);
        };
        auto fetch_v = [&](E (&v)[4], int c) {
            const int tb = min(c * C + m * 16 + rl, T - 1);   // rows past the prompt read its last token
            const E* src = vg + ((size_t)b * p.Ts + p.t0 + tb) * Hv * DV;
            if constexpr (sizeof(E) == 2) {
                const uint2 u = *reinterpret_cast<const uint2*>(src);
                __builtin_memcpy(v, &u, 8);
            } else {
                const float4 u = *reinterpret_cast<const float4*>(src);
                __builtin_memcpy(v, &u, 16);
            }
        };
        auto fetch_k = [&](COps& op, int c) {
            const float* gc = gates + (size_t)c * Sh::GATES;
            op.gn = gc[2 * C];
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                const int dt = min(w4 + 4 * tw, DT - 1);
                const E* zsrc = Zg + (size_t)c * Sh::Z_PER_CHUNK + (size_t)dt * NKC * Sh::FRAG;
#pragma unroll
                for (int kb = 0; kb < NKC; kb += X::GRP) X::ld_grp(zsrc + X::foff(kb, lane), &op.z[tw][kb]);
            }
        };
        auto fetch = [&](COps& op, int c) { fetch_w(op, c); fetch_k(op, c); };

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
        auto step = [&](COps& op, E (&v)[4], int c, int nc, int nvc, auto pftag, auto vftag) {
            constexpr bool PF = decltype(pftag)::value, VF = decltype(vftag)::value;
            // keeps the next step's operand uses (and so their waits) out of this one
            __builtin_amdgcn_sched_barrier(0);
            const int cur = c & 1;
            if (has_tile) {
                const E* sr = &Sb[cur][rl * LDS_];
                const E* sl = &Sl[cur][SPLIT ? rl * LDS_ : 0];
                typename X::frag sh[NKD], slo[NKD];
#pragma unroll
                for (int kb = 0; kb < NKD; kb += X::GRP) {
                    X::ld_grp(sr + X::doff(kb, g), &sh[kb]);
                    if (SPLIT) X::ld_grp(sl + X::doff(kb, g), &slo[kb]);
                }
                // (K S^T)^T = S K^T: the state rows as A and the K rows as B (the same fragments
                // in the other operand order), so that lane (g, t) ends with the state rows
                // rq..rq+3 of token t, whose v is 8 (fp32: 16) contiguous bytes
                f32x4 acc = zero4(), accl = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) {
                    acc = X::mma(sh[kb], op.kf[kb], acc);
                    if (SPLIT) accl = X::mma(slo[kb], op.kf[kb], accl);
                }
                if (SPLIT) acc += accl;
                E y[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = X::from_f(X::to_f(v[j]) - op.gk * acc[j]);
#pragma unroll
                for (int j = 0; j < 4; ++j) YT[(rq + j) * LDU + m * 16 + rl] = y[j];
            }
            if (PF) fetch_w(op, nc);
            lds_barrier();   // (B1) Y complete; chunk c's slice was read from buffer cur
            if (VF) fetch_v(v, nvc);
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) {
                const int dt = w4 + 4 * tw;
                if (dt < DT) {
                    f32x4 acc = St[tw] * op.gn;
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        acc = X::mma(op.z[tw][kb], X::ld_perm(YT + rl * LDU + X::poff(kb, g)), acc);
                    St[tw] = acc;
                }
            }
            if (PF) fetch_k(op, nc);
            publish(cur ^ 1);
            lds_barrier();   // (B2) next slice published; output waves are done with Y
        };

        publish(0);
        COps op[NBC];
        E vb[NBV][4];
        // first fetches in the order the loop issues them (each operand set's K rows, then the v
        // set NBV - NBC later, then the set's Z), so that the outstanding loads stand in the same order when the
        // loop is entered as when it repeats, and the waits at its head stay exact
        // (the scheduling barriers keep the compiler from regrouping them)
        auto prologue = [&] {
#pragma unroll
            for (int j = 0; j < NBV - NBC; ++j) {
                fetch_v(vb[j], min(j, N - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < NBC; ++j) {
                fetch_w(op[j], min(j, N - 1));
                __builtin_amdgcn_sched_barrier(0);
                fetch_v(vb[NBV - NBC + j], min(NBV - NBC + j, N - 1));
                __builtin_amdgcn_sched_barrier(0);
                fetch_k(op[j], min(j, N - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
            lds_barrier();
        };
        // the last chunks after c, fewer than NBV: the v sets hold all of them, the operand sets
        // the next NBC, refilled while chunks remain
        std::true_type yes;
        std::false_type no;
        auto remainder = [&](int c) {
#pragma unroll
            for (int j = 0; j < NBV; ++j) {
                if (c + j >= N) break;
                if (c + j + NBC < N) step(op[j % NBC], vb[j], c + j, c + j + NBC, 0, yes, no);
                else step(op[j % NBC], vb[j], c + j, 0, 0, no, no);
            }
        };
        // The loop runs whole passes of NBV chunks only: a pass that could stop part-way would
        // let the waits at the loop's head assume the last loads of a cut-short pass are the
        // newest.  Prompts shorter than one pass take a separate path, so that no operand set
        // has to live across the loop into the remainder (which made the compiler spill them).
        if (N >= NBV) {
            prologue();
            int c = 0;
            do {
#pragma unroll
                for (int j = 0; j < NBV; ++j)
                    step(op[j % NBC], vb[j], c + j, min(c + j + NBC, N - 1), min(c + j + NBV, N - 1), yes, yes);
                c += NBV;
            } while (c + NBV <= N);
            remainder(c);
        } else {
            prologue();
            remainder(0);
        }

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
        const int pkmax = (m * 16 + 15) / KB;   // last k-block of P row tile m with nonzeros
        const E* qfg = reinterpret_cast<const E*>(p.QF) + ((size_t)b * Hk + hk) * N * Sh::W_PER_CHUNK
                       + (size_t)m * NKD * Sh::FRAG;
        E* og = reinterpret_cast<E*>(p.o) + (size_t)h * DV + i0;

        auto fetch = [&](OOps& op, int c) {
            const int t0 = c * C;
            op.gr = gates[(size_t)c * Sh::GATES + m * 16 + rl];
            const E* qsrc = qfg + (size_t)c * Sh::W_PER_CHUNK;
#pragma unroll
            for (int kb = 0; kb < NKD; kb += X::GRP) X::ld_grp(qsrc + X::foff(kb, lane), &op.q[kb]);
            const E* psrc = Pg + (size_t)c * Sh::P_PER_CHUNK + (size_t)m * NKC * Sh::FRAG;
            // k-blocks past the diagonal are zero, not stored (an fp32 group of four k-blocks
            // is one 16-token tile, wholly on one side of it)
#pragma unroll
            for (int kb = 0; kb < NKC; kb += X::GRP) {
                if (kb <= pkmax) {
                    X::ld_grp(psrc + X::foff(kb, lane), &op.p[kb]);
                } else {
#pragma unroll
                    for (int i = 0; i < X::GRP; ++i) op.p[kb + i] = X::zero();
                }
            }
        };
        auto step = [&](const OOps& op, int c, auto tailtag) {
            constexpr bool TAIL = decltype(tailtag)::value;
            __builtin_amdgcn_sched_barrier(0);
            const int t0 = c * C;
            lds_barrier();   // (B1) Y of chunk c is in LDS; buffer (c & 1) holds chunk c's slice
            if (has_tile) {
                const E* sr = &Sb[c & 1][rl * LDS_];
                const bool qok = !TAIL || (t0 + m * 16 + rl < T);
                // The output tile transposed, O^T = S Q^T + Y^T P'^T: the same fragments as operands
                // in the other order (the state rows and Y rows as A, the Q and P' rows as B), so
                // that lane (g, t) ends with the state rows rq..rq+3 of token t -- contiguous in o
                // and stored from the accumulator directly, with the nontemporal hint (o is
                // written once and not read here)
                f32x4 accq = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; kb += X::GRP) {
                    frag sh[X::GRP];
                    X::ld_grp(sr + X::doff(kb, g), sh);
#pragma unroll
                    for (int i = 0; i < X::GRP; ++i)
                        accq = X::mma(sh[i], TAIL ? X::keep_if(op.q[kb + i], qok) : op.q[kb + i], accq);
                }
                f32x4 acc = accq * op.gr;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)   // P fragments: tokens in the permuted order
                    if (kb <= pkmax) acc = X::mma(X::ld_perm(YT + rl * LDU + X::poff(kb, g)), op.p[kb], acc);
                const int t = t0 + m * 16 + rl;
                if (!TAIL || t < T) {
                    E* dst = og + ((size_t)b * p.Ts + p.t0 + t) * Hv * DV + rq;
                    if constexpr (sizeof(E) == 2) {
                        const u32x2 w = {f2bf2(acc[0], acc[1]), f2bf2(acc[2], acc[3])};
                        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(dst));
                    } else {
                        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(dst));
                    }
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

// Workgroups of the intra kernel that fit on the current device at once (the kernel loops
// over its work items, so it is launched with exactly that many), cached per device.
template <typename E, int DK, int DV, int C, bool NORM>
inline int intra_capacity() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int cap = cache[dev].load(std::memory_order_relaxed);
    if (cap == 0) {
        int ncu = 0, per = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) ncu = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, intra_chunk_kernel<E, DK, DV, C, NORM>, kThreads, 0) !=
            hipSuccess)
            per = 1;
        cap = std::max(1, ncu) * std::max(1, per);
        cache[dev].store(cap, std::memory_order_relaxed);
    }
    return cap;
}

// stage bit 1: intra-chunk kernel; bit 2: inter-chunk kernel.
template <typename E, int DK, int DV, int C>
inline hipError_t launch_prefill(const PrefillParams& p, int stages, hipStream_t stream) {
    if (stages & 1) {
        // grid: a multiple of 8 (Hv / Hk) workgroups (see the work-item order), at most the
        // resident capacity and at most the number of work items
        const int unit = 8 * (p.Hv / p.Hk);
        const int nitems = (p.B * p.N * p.Hk + 7) / 8 * 8 * (p.Hv / p.Hk);
        auto go = [&](auto norm) {
            constexpr bool NORM = decltype(norm)::value;
            const int cap = intra_capacity<E, DK, DV, C, NORM>();
            const int grid = std::min(nitems, std::max(unit, cap / unit * unit));
            return launch_kernel(intra_chunk_kernel<E, DK, DV, C, NORM>, dim3(grid), dim3(kThreads),
                                 stream, p);
        };
        const hipError_t e = p.qk_norm ? go(std::true_type{}) : go(std::false_type{});
        if (e != hipSuccess) return e;
    }
    if (stages & 2) {
        const dim3 g2(p.B * p.Hv * (DV / 16));
        return launch_kernel(inter_chunk_kernel<E, DK, DV, C, sizeof(E) == 2>, g2, dim3(kScanThreads),
                             stream, p);
    }
    return hipSuccess;
}

}  // namespace gdn
