// gdn_decode.h -- one-token recurrent update (decode step) of the gated delta rule.
//
// "Optimizing on-device inference for Apple Silicon", section "Decode: minimise bytes
// moved per token": at batch 1 the step is bound by the bytes it moves, and section
// "Reduce intermediate and state traffic" fuses the recurrent update into one kernel
// that keeps temporaries in registers.  Here the state is the traffic: every fp32
// element is read once and written once, nothing else touches memory in bulk.
//
// Per state row i (rows evolve independently):
//   s_k = S_i . k,  s_q = S_i . q                  (cross-lane reductions)
//   delta_i = beta (v_i - a s_k)                   a = exp(g)
//   S_i <- a S_i + delta_i k^T
//   o_i = S_i(new) . q = a s_q + delta_i (k . q)
// With fused normalisation q and k are first scaled to unit length (each lane group of a
// row reduces the squared norm with the same shuffles as the dot products).
//
// Mapping: a row of dk floats is read by dk/4 consecutive lanes as 16-byte vectors, so
// a wavefront reads 1 KiB of contiguous state per instruction; each thread keeps NIT
// rows in flight before it reduces.  The state is read and written with the nontemporal
// hint (it is touched once per step).  No matrix cores: the arithmetic is 3 FMAs per state
// element against 8 bytes of traffic.
#pragma once

#include "gdn_device.h"

namespace gdn {

struct DecodeParams {
    const void* q;        // [B][Hk][DK]
    const void* k;        // [B][Hk][DK]
    const void* v;        // [B][Hv][DV]
    const float* g;       // [B][Hv]
    const float* beta;    // [B][Hv]
    const float* state_in;
    float* state_out;     // [B][Hv][DV][DK]
    void* o;              // [B][Hv][DV]
    int B, Hk, Hv;
    int qk_norm;          // nonzero: q and k are L2-normalised per head first
};

// Per-layer pointers of a launch over several independent layers (one decode token through
// a layer stack); the sizes and flags are shared.  Passed by value as a kernel argument, so a
// launch needs no device memory for it.
constexpr int kDecodeLayersPerLaunch = 32;
struct DecodeLayerPtrs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* state_in;
    float* state_out;
    void* o;
};
struct DecodeTable {
    DecodeLayerPtrs layer[kDecodeLayersPerLaunch];
    int nlayers, B, Hk, Hv;
    int qk_norm;
};

// Tiling of a decode workgroup (256 threads): LPR lanes per state row, RIT rows per pass of
// the workgroup, RPB rows per workgroup (NIT passes, each thread's loads all in flight at once),
// NBLK workgroups per (batch, value head).  Four passes instead of two measured the same.
template <int DK, int DV>
struct DecodeTiling {
    static constexpr int LPR = DK / 4;
    static constexpr int RIT = 256 / LPR;
    static constexpr int RPB = (2 * RIT < DV) ? 2 * RIT : DV;
    static constexpr int NIT = RPB / RIT;
    static constexpr int NBLK = DV / RPB;
};

// One workgroup's share of a decode step: block `wg` of the B * Hv * NBLK blocks of p.
template <typename E, int DK, int DV>
__device__ __forceinline__ void decode_block(const DecodeParams& p, int wg) {
    using X = Elem<E>;
    typedef DecodeTiling<DK, DV> Tl;
    constexpr int LPR = Tl::LPR, RIT = Tl::RIT, RPB = Tl::RPB, NIT = Tl::NIT, NBLK = Tl::NBLK;
    static_assert(RIT <= DV && NIT * RIT == RPB && NBLK * RPB == DV, "decode tiling");

    const int blk = wg % NBLK;
    const int bh = wg / NBLK;
    const int h = bh % p.Hv, b = bh / p.Hv;
    const int hk = h / (p.Hv / p.Hk);
    const int tid = threadIdx.x;
    const int sub = tid % LPR, rloc = tid / LPR;
    const int c0 = sub * 4;

    // Every global load is issued before the first use, so the whole step costs one memory
    // round trip: the state rows, this thread's v elements, q, k, g and beta.
    const size_t row0 = ((size_t)b * p.Hv + h) * DV + (size_t)blk * RPB + rloc;
    float4 s[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it)
        s[it] = ld_stream4(p.state_in + (row0 + (size_t)it * RIT) * DK + c0);
    const E* vp = reinterpret_cast<const E*>(p.v);
    E vr[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) vr[it] = vp[row0 + (size_t)it * RIT];
    const E* kp = reinterpret_cast<const E*>(p.k) + ((size_t)b * p.Hk + hk) * DK + c0;
    const E* qp = reinterpret_cast<const E*>(p.q) + ((size_t)b * p.Hk + hk) * DK + c0;
    E kraw[4], qraw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { kraw[e] = kp[e]; qraw[e] = qp[e]; }
    const float graw = p.g[(size_t)b * p.Hv + h];
    const float bt = p.beta[(size_t)b * p.Hv + h];

    float kk[4], qq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { kk[e] = X::to_f(kraw[e]); qq[e] = X::to_f(qraw[e]); }
    if (p.qk_norm) {   // the LPR lanes of a row hold the whole vector between them
        const float ssk = group_sum<LPR>(kk[0] * kk[0] + kk[1] * kk[1] + kk[2] * kk[2] + kk[3] * kk[3]);
        const float ssq = group_sum<LPR>(qq[0] * qq[0] + qq[1] * qq[1] + qq[2] * qq[2] + qq[3] * qq[3]);
        const float ik = rsqrtf(ssk + kNormEps), iq = rsqrtf(ssq + kNormEps);
#pragma unroll
        for (int e = 0; e < 4; ++e) { kk[e] *= ik; qq[e] *= iq; }
    }
    const float a = expf(graw);
    const float kq = group_sum<LPR>(kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3]);

    E* op = reinterpret_cast<E*>(p.o);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const float sk = group_sum<LPR>(s[it].x * kk[0] + s[it].y * kk[1] + s[it].z * kk[2] + s[it].w * kk[3]);
        const float sq = group_sum<LPR>(s[it].x * qq[0] + s[it].y * qq[1] + s[it].z * qq[2] + s[it].w * qq[3]);
        const size_t row = row0 + (size_t)it * RIT;
        const float delta = bt * (X::to_f(vr[it]) - a * sk);
        float4 ns;
        ns.x = a * s[it].x + delta * kk[0];
        ns.y = a * s[it].y + delta * kk[1];
        ns.z = a * s[it].z + delta * kk[2];
        ns.w = a * s[it].w + delta * kk[3];
        st_stream4(p.state_out + row * DK + c0, ns);
        if (sub == 0) op[row] = X::from_f(a * sq + delta * kq);
    }
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    decode_block<E, DK, DV>(p, blockIdx.x);
}

// The same step over t.nlayers layers in one launch: workgroup (w, l) of the 2-D grid takes
// block w of layer l, so every layer's state is read and written exactly as by its own
// decode_kernel launch (the layer index needs no division by sizes loaded from the arguments,
// so the layer's pointers are fetched at once).
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void decode_layers_kernel(DecodeTable t) {
    const int l = blockIdx.y;
    const int w = blockIdx.x;
    const DecodeLayerPtrs& lp = t.layer[l];
    DecodeParams p;
    p.q = lp.q; p.k = lp.k; p.v = lp.v; p.g = lp.g; p.beta = lp.beta;
    p.state_in = lp.state_in; p.state_out = lp.state_out; p.o = lp.o;
    p.B = t.B; p.Hk = t.Hk; p.Hv = t.Hv; p.qk_norm = t.qk_norm;
    decode_block<E, DK, DV>(p, w);
}

template <typename E, int DK, int DV>
inline hipError_t launch_decode_layers(const DecodeTable& t, hipStream_t stream) {
    const dim3 grid((unsigned)(t.B * t.Hv * DecodeTiling<DK, DV>::NBLK), (unsigned)t.nlayers);
    return launch_kernel(decode_layers_kernel<E, DK, DV>, grid, dim3(256), stream, t);
}

template <typename E, int DK, int DV>
inline hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)(p.B * p.Hv * DecodeTiling<DK, DV>::NBLK));
    return launch_kernel(decode_kernel<E, DK, DV>, grid, dim3(256), stream, p);
}

}  // namespace gdn
