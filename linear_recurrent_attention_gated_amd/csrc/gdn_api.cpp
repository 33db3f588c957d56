// gdn_api.cpp -- the C ABI declared in include/gdn.h: synchronous argument validation,
// workspace carving, and dispatch to the compiled kernel variants.  Nothing here
// allocates device memory or synchronises the stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }
size_t elem_size(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Span {
    const void* p;
    size_t n;
};
bool overlap(Span a, Span b) {
    if (!a.p || !b.p || !a.n || !b.n) return false;
    const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
    return x < y + b.n && y < x + a.n;
}
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Longest prompt for which GDN_PATH_AUTO takes the token-sequential path: the crossover of the
// two prefill forms measured on MI355X (cold calls, chunk 64), where their times cross.
//   dk = dv:        32     64    128
//   bf16 operands:  43     42     42      (the same at 4 and 32 value heads, batch 1)
//   fp32 operands:  89     96    110
// The token-sequential form holds a state row on 16 lanes; up to 1,024 waves (one per SIMD)
// its time per token does not depend on the rows, and the crossover does not either.  Above
// that its time grows with the rows while the blockwise form's short-prompt time barely does:
// at batch 4, 32 value heads, d = 128 (4,096 waves) the crossings were 24 (bf16) and 46
// (fp32), a power law in the waves with exponents 0.42 and 0.66 (bf16 at d = 64, 2,048 waves:
// 28 measured, 31 by the law).  Between the tabulated
// dk * dv the crossover is interpolated in log2(dk * dv).
int sequential_max_tokens(int B, int Hv, int dk, int dv, gdn_dtype dtype) {
    static const double kBf16[3] = {43.0, 42.0, 42.0}, kF32[3] = {89.0, 96.0, 110.0};
    const double* t = dtype == GDN_BF16 ? kBf16 : kF32;
    const double x = std::log2((double)dk * dv);   // 10 .. 14
    double t1 = x <= 12.0 ? t[0] + (t[1] - t[0]) * (x - 10.0) / 2.0 : t[1] + (t[2] - t[1]) * (x - 12.0) / 2.0;
    const double waves = (double)B * Hv * dv * 16 / 64.0;
    if (waves > 1024.0) t1 *= std::pow(1024.0 / waves, dtype == GDN_BF16 ? 0.42 : 0.66);
    return t1 < 1.0 ? 1 : (int)t1;
}

// Last-level-cache budget of one blockwise prefill pass: its workspace plus its v rows (what the
// scan reads after the intra-chunk kernel has written or touched it).  MI355X has 256 MB of
// last-level cache; measured there (16/32 heads, d = 128, cold): bf16 prompts of up to 6,144
// tokens (~176 MB) run fastest in one pass, longer ones in equal passes of at most that many
// (8K: 195 against 252 us in one pass; 128K: 2.9 against 3.5 ms; batch 2 at 4K: 217 against
// 259 us).  fp32 passes lose less to cache misses (their scan is slower per chunk) and more to
// each pass's fixed cost: 4-16K-token passes are 5-14% faster than one pass at 16-32K tokens,
// but two passes of 2K tokens at batch 2 are 8% slower than one, so its budget is larger.
size_t pass_cache_budget(gdn_dtype dtype) {
    return dtype == GDN_BF16 ? ((size_t)176 << 20) : ((size_t)600 << 20);
}

// Workspace regions of the blockwise prefill (see gdn_prefill.h).
struct Layout {
    size_t KF, QF, Z, P, gam, total;
};
Layout layout(int B, int T, int Hk, int Hv, int dk, int /*dv*/, int chunk, gdn_dtype dt) {
    const size_t es = elem_size(dt);
    const size_t N = ((size_t)T + chunk - 1) / chunk, Tp = N * (size_t)chunk;
    // token-side k-blocks of the MFMA fragments are padded to 32 (bf16) / 4 (fp32) tokens
    const size_t kb = dt == GDN_BF16 ? 32 : 4;
    const size_t cp = ((size_t)chunk + kb - 1) / kb * kb;
    Layout L;
    size_t off = 0;
    L.KF = off;  off = round_up(off + (size_t)B * Hk * Tp * dk * es, 256);
    L.QF = off;  off = round_up(off + (size_t)B * Hk * Tp * dk * es, 256);
    L.Z = off;   off = round_up(off + (size_t)B * Hv * N * dk * cp * es, 256);
    L.P = off;   off = round_up(off + (size_t)B * Hv * Tp * cp * es, 256);
    L.gam = off; off = round_up(off + (size_t)B * Hv * N * (2 * chunk + 4) * sizeof(float), 256);
    L.total = off;
    return L;
}

gdn_status shape_check(int B, int T, int Hk, int Hv, int dk, int dv, int chunk, gdn_dtype dt,
                       bool prefill) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || Hv % Hk != 0) return GDN_ERR_SHAPE;
    if (dt != GDN_BF16 && dt != GDN_F32) return GDN_ERR_UNSUPPORTED;
    if (!supported_dim(dk) || !supported_dim(dv)) return GDN_ERR_UNSUPPORTED;
    if (prefill && !supported_chunk(chunk)) return GDN_ERR_UNSUPPORTED;
    // keep every launch dimension and 32-bit intermediate in range
    if ((int64_t)B * Hv * (dv / 16) > INT32_MAX / 2 || (int64_t)T > (int64_t)INT32_MAX / 4)
        return GDN_ERR_SHAPE;
    if (prefill && (Hv > 65535 || B > 65535)) return GDN_ERR_SHAPE;
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_prefill_workspace_bytes(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                   gdn_dtype dtype) {
    if (shape_check(B, T, Hk, Hv, dk, dv, chunk, dtype, true) != GDN_OK || T == 0) return 0;
    return layout(B, T, Hk, Hv, dk, dv, chunk, dtype).total;
}

}  // extern "C"

// ---- allocation-free prefill ------------------------------------------------------------
// The workspace of gdn_prefill_noalloc: a file-scope device array, one copy per GPU, held until
// the process ends.  In host code `scratch` only names the symbol; its device address comes
// from hipGetSymbolAddress, once per device (with that device current), and only that address
// is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
gdn_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return GDN_OK;
}

}  // namespace

namespace {

// How a prefill call is evaluated once its arguments are checked: the blockwise form (the
// workspace path), the token-sequential form, or (one token from a given state) the decode step.
enum class Form { blockwise, sequential, decode_step };

gdn_status prefill_stages(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, void* o, float* state_out,
                          int B, int T, int Hk, int Hv, int dk, int dv, int chunk, gdn_dtype dtype,
                          void* workspace, size_t workspace_bytes, void* stream, int stages,
                          int qk_norm, Form form, bool noalloc = false) {
    const gdn_status sc = shape_check(B, T, Hk, Hv, dk, dv, chunk, dtype, true);
    if (sc != GDN_OK) return sc;
    if (!state_out) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    const size_t es = elem_size(dtype);
    const size_t nqk = (size_t)B * T * Hk * dk * es, nv = (size_t)B * T * Hv * dv * es;
    const size_t ng = (size_t)B * T * Hv * sizeof(float);
    const size_t ns = (size_t)B * Hv * dv * dk * sizeof(float);
    if (!aligned(state_out, 16) || (state_in && !aligned(state_in, 16))) return GDN_ERR_ALIGN;
    if (T > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(g, 4) || !aligned(beta, 4))
            return GDN_ERR_ALIGN;
    }
    const Span sq{q, T ? nqk : 0}, sk{k, T ? nqk : 0}, sv{v, T ? nv : 0}, sg{g, T ? ng : 0},
        sb{beta, T ? ng : 0}, si{state_in, ns}, so{o, T ? nv : 0}, ss{state_out, ns},
        sw{workspace, T ? workspace_bytes : 0};
    for (Span in : {sq, sk, sv, sg, sb, si, sw})
        if (overlap(so, in)) return GDN_ERR_ALIAS;
    for (Span in : {sq, sk, sv, sg, sb, sw, so})
        if (overlap(ss, in)) return GDN_ERR_ALIAS;
    if (state_in && state_in != state_out && overlap(ss, si)) return GDN_ERR_ALIAS;
    for (Span in : {sq, sk, sv, sg, sb, si})
        if (overlap(sw, in)) return GDN_ERR_ALIAS;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (T == 0) {
        if (!(stages & 2)) return GDN_OK;
        return gdn::copy_state(state_in, state_out, (size_t)B * Hv * dv * dk, st) == hipSuccess
                   ? GDN_OK : GDN_ERR_HIP;
    }
    if (form == Form::decode_step) {   // (T == 1, state_in given) its layouts are the prefill's at T = 1
        gdn::DecodeParams p;
        p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.state_in = state_in;
        p.state_out = state_out; p.o = o; p.B = B; p.Hk = Hk; p.Hv = Hv; p.qk_norm = qk_norm;
        const hipError_t e = dtype == GDN_BF16 ? gdn::decode_bf16(dk, dv, p, st) : gdn::decode_f32(dk, dv, p, st);
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    if (form == Form::sequential) {   // the state stays in registers: no workspace, one launch
        gdn::PrefillParams p{};
        p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.state_in = state_in;
        p.o = o; p.state_out = state_out;
        p.B = B; p.T = T; p.Hk = Hk; p.Hv = Hv; p.N = 0; p.Ts = T; p.t0 = 0; p.qk_norm = qk_norm;
        const hipError_t e = dtype == GDN_BF16 ? gdn::sequential_bf16(dk, dv, p, st)
                                               : gdn::sequential_f32(dk, dv, p, st);
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    if (noalloc) {   // every argument has been validated: now (only) look up the array
        if (layout(B, chunk, Hk, Hv, dk, dv, chunk, dtype).total > GDN_NOALLOC_SCRATCH_BYTES)
            return GDN_ERR_WORKSPACE;
        const gdn_status sa = scratch_address(&workspace);
        if (sa != GDN_OK) return sa;
        workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace) return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
    // Tokens per pass.  The stages alone need the one-pass workspace.  The full prefill runs the
    // prompt in passes of whole chunks, carrying the state through state_out, when the workspace
    // does not hold it in one, or when one pass would not keep its working set in the last-level
    // cache (pass_cache_budget); the passes are then of equal length.
    int seg = T;
    const int nchunks = (T + chunk - 1) / chunk;
    if (stages != 3) {
        if (layout(B, T, Hk, Hv, dk, dv, chunk, dtype).total > workspace_bytes) return GDN_ERR_WORKSPACE;
    } else {
        const size_t budget = pass_cache_budget(dtype);
        // longest pass (in chunks) that satisfies pred, at most the whole prompt; 0 if none does
        auto longest = [&](auto pred) {
            if (pred(nchunks)) return nchunks;
            int lo = 0, hi = nchunks;   // pred(lo) holds (or lo = 0), pred(hi) does not
            while (hi - lo > 1) {
                const int mid = (lo + hi) / 2;
                if (pred(mid)) lo = mid;
                else hi = mid;
            }
            return lo;
        };
        const int ws_max = longest([&](int n) {
            return layout(B, n * chunk, Hk, Hv, dk, dv, chunk, dtype).total <= workspace_bytes;
        });
        if (ws_max == 0) return GDN_ERR_WORKSPACE;
        // passes shorter than ~512 tokens would pay their fixed cost for little: when the
        // budget holds fewer (many heads or batches), the cache is not a reason to split
        int cache_max = longest([&](int n) {
            return layout(B, n * chunk, Hk, Hv, dk, dv, chunk, dtype).total +
                       (size_t)B * n * chunk * Hv * dv * es <= budget;
        });
        if (cache_max * chunk < 512) cache_max = nchunks;
        const int cap = std::min(ws_max, cache_max);
        if (cap < nchunks) {
            const int npass = (nchunks + cap - 1) / cap;
            seg = (nchunks + npass - 1) / npass * chunk;
        }
    }

    for (int t0 = 0; t0 < T; t0 += seg) {
        const int Tp = T - t0 < seg ? T - t0 : seg;
        const Layout L = layout(B, Tp, Hk, Hv, dk, dv, chunk, dtype);
        gdn::PrefillParams p;
        p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
        p.state_in = t0 == 0 ? state_in : state_out;
        p.o = o; p.state_out = state_out;
        char* ws = static_cast<char*>(workspace);
        p.KF = ws + L.KF; p.QF = ws + L.QF; p.Z = ws + L.Z; p.P = ws + L.P;
        p.gam = reinterpret_cast<float*>(ws + L.gam);
        p.B = B; p.T = Tp; p.Hk = Hk; p.Hv = Hv; p.N = (Tp + chunk - 1) / chunk;
        p.Ts = T; p.t0 = t0;
        p.qk_norm = qk_norm;

        hipError_t e = hipErrorInvalidValue;
        if (dtype == GDN_BF16) {
            if (chunk == 16) e = gdn::prefill_bf16_c16(dk, dv, p, stages, st);
            else if (chunk == 32) e = gdn::prefill_bf16_c32(dk, dv, p, stages, st);
            else e = gdn::prefill_bf16_c64(dk, dv, p, stages, st);
        } else {
            if (chunk == 16) e = gdn::prefill_f32_c16(dk, dv, p, stages, st);
            else if (chunk == 32) e = gdn::prefill_f32_c32(dk, dv, p, stages, st);
            else e = gdn::prefill_f32_c64(dk, dv, p, stages, st);
        }
        if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* state_in, void* o, float* state_out,
                       int B, int T, int Hk, int Hv, int dk, int dv, int chunk, gdn_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_stages(q, k, v, g, beta, state_in, o, state_out, B, T, Hk, Hv, dk, dv, chunk,
                          dtype, workspace, workspace_bytes, stream, 3, 0, Form::blockwise);
}

gdn_status gdn_prefill_ex(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* state_in, void* o, float* state_out,
                          int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                          gdn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                          unsigned flags) {
    if (flags & ~(unsigned)(GDN_QK_NORM | GDN_PATH_SEQUENTIAL | GDN_PATH_AUTO) ||
        ((flags & GDN_PATH_SEQUENTIAL) && (flags & GDN_PATH_AUTO)))
        return GDN_ERR_UNSUPPORTED;
    Form form = (flags & GDN_PATH_SEQUENTIAL) ? Form::sequential : Form::blockwise;
    if (flags & GDN_PATH_AUTO) {
        // one token from a given state: the decode step, a single read and write of the state;
        // else the sequential form up to the measured crossover
        if (T == 1 && state_in) form = Form::decode_step;
        else if (T <= gdn_prefill_sequential_max_tokens(B, Hk, Hv, dk, dv, dtype)) form = Form::sequential;
    }
    return prefill_stages(q, k, v, g, beta, state_in, o, state_out, B, T, Hk, Hv, dk, dv, chunk,
                          dtype, workspace, workspace_bytes, stream, 3,
                          (flags & GDN_QK_NORM) ? 1 : 0, form);
}

int gdn_prefill_sequential_max_tokens(int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype) {
    if (shape_check(B, 1, Hk, Hv, dk, dv, 16, dtype, true) != GDN_OK) return 0;
    return sequential_max_tokens(B, Hv, dk, dv, dtype);
}

gdn_status gdn_prefill_qknorm(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* state_in, void* o,
                              float* state_out, int B, int T, int Hk, int Hv, int dk, int dv,
                              int chunk, gdn_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return prefill_stages(q, k, v, g, beta, state_in, o, state_out, B, T, Hk, Hv, dk, dv, chunk,
                          dtype, workspace, workspace_bytes, stream, 3, 1, Form::blockwise);
}

gdn_status gdn_prefill_prepare(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* state_in, void* o,
                               float* state_out, int B, int T, int Hk, int Hv, int dk, int dv,
                               int chunk, gdn_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return prefill_stages(q, k, v, g, beta, state_in, o, state_out, B, T, Hk, Hv, dk, dv, chunk,
                          dtype, workspace, workspace_bytes, stream, 1, 0, Form::blockwise);
}

gdn_status gdn_prefill_scan(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* state_in, void* o, float* state_out,
                            int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                            gdn_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return prefill_stages(q, k, v, g, beta, state_in, o, state_out, B, T, Hk, Hv, dk, dv, chunk,
                          dtype, workspace, workspace_bytes, stream, 2, 0, Form::blockwise);
}

gdn_status gdn_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* state_in, void* o, float* state_out,
                               int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                               gdn_dtype dtype, void* stream) {
    return prefill_stages(q, k, v, g, beta, state_in, o, state_out, B, T, Hk, Hv, dk, dv, chunk,
                          dtype, nullptr, 0, stream, 3, 0, Form::blockwise, true);
}

}  // extern "C"

namespace {

// The spans of one decode step's tensors: q, k, v, g, beta, state_in (inputs), state_out, o.
struct DecodeSpans {
    Span in[6], ss, so;
};
DecodeSpans decode_spans(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* state_in, float* state_out, void* o,
                         int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype) {
    const size_t es = elem_size(dtype);
    DecodeSpans d;
    d.in[0] = {q, (size_t)B * Hk * dk * es};
    d.in[1] = {k, (size_t)B * Hk * dk * es};
    d.in[2] = {v, (size_t)B * Hv * dv * es};
    d.in[3] = {g, (size_t)B * Hv * 4};
    d.in[4] = {beta, (size_t)B * Hv * 4};
    d.in[5] = {state_in, (size_t)B * Hv * dv * dk * 4};
    d.ss = {state_out, (size_t)B * Hv * dv * dk * 4};
    d.so = {o, (size_t)B * Hv * dv * es};
    return d;
}

// Pointer, alignment and overlap rules of one decode step (sizes already checked).
gdn_status decode_check(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* state_in, float* state_out, void* o, int B,
                        int Hk, int Hv, int dk, int dv, gdn_dtype dtype) {
    if (!q || !k || !v || !g || !beta || !state_in || !state_out || !o) return GDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(state_in, 16) || !aligned(state_out, 16) || !aligned(g, 4) || !aligned(beta, 4))
        return GDN_ERR_ALIGN;
    const DecodeSpans d = decode_spans(q, k, v, g, beta, state_in, state_out, o, B, Hk, Hv, dk, dv, dtype);
    for (const Span& in : d.in)
        if (overlap(d.so, in)) return GDN_ERR_ALIAS;
    if (overlap(d.so, d.ss)) return GDN_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        if (overlap(d.ss, d.in[i])) return GDN_ERR_ALIAS;
    if (state_in != state_out && overlap(d.ss, d.in[5])) return GDN_ERR_ALIAS;
    return GDN_OK;
}

gdn_status decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* state_in, float* state_out, void* o, int B, int Hk, int Hv, int dk,
                  int dv, gdn_dtype dtype, void* stream, int qk_norm) {
    const gdn_status sc = shape_check(B, 1, Hk, Hv, dk, dv, 16, dtype, false);
    if (sc != GDN_OK) return sc;
    const gdn_status pc = decode_check(q, k, v, g, beta, state_in, state_out, o, B, Hk, Hv, dk, dv, dtype);
    if (pc != GDN_OK) return pc;

    gdn::DecodeParams p;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.state_in = state_in;
    p.state_out = state_out; p.o = o; p.B = B; p.Hk = Hk; p.Hv = Hv; p.qk_norm = qk_norm;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = dtype == GDN_BF16 ? gdn::decode_bf16(dk, dv, p, st) : gdn::decode_f32(dk, dv, p, st);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

extern "C" {

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* state_in, float* state_out, void* o,
                           int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype, void* stream) {
    return decode(q, k, v, g, beta, state_in, state_out, o, B, Hk, Hv, dk, dv, dtype, stream, 0);
}

gdn_status gdn_decode_step_qknorm(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const float* state_in, float* state_out,
                                  void* o, int B, int Hk, int Hv, int dk, int dv, gdn_dtype dtype,
                                  void* stream) {
    return decode(q, k, v, g, beta, state_in, state_out, o, B, Hk, Hv, dk, dv, dtype, stream, 1);
}

gdn_status gdn_decode_step_layers(const gdn_decode_layer* layers, int nlayers, int B, int Hk,
                                  int Hv, int dk, int dv, gdn_dtype dtype, unsigned flags,
                                  void* stream) {
    if (!layers) return GDN_ERR_NULL;
    if (nlayers < 1) return GDN_ERR_SHAPE;
    if (flags & ~(unsigned)GDN_QK_NORM) return GDN_ERR_UNSUPPORTED;
    const gdn_status sc = shape_check(B, 1, Hk, Hv, dk, dv, 16, dtype, false);
    if (sc != GDN_OK) return sc;
    if ((int64_t)nlayers * B * Hv * (dv / 16) > INT32_MAX / 2) return GDN_ERR_SHAPE;
    for (int l = 0; l < nlayers; ++l) {
        const gdn_decode_layer& L = layers[l];
        const gdn_status pc = decode_check(L.q, L.k, L.v, L.g, L.beta, L.state_in, L.state_out,
                                           L.o, B, Hk, Hv, dk, dv, dtype);
        if (pc != GDN_OK) return pc;
    }
    // the layers run concurrently: no output of one layer may overlap any tensor of another
    for (int l = 0; l < nlayers; ++l) {
        const gdn_decode_layer& L = layers[l];
        const DecodeSpans a = decode_spans(L.q, L.k, L.v, L.g, L.beta, L.state_in, L.state_out, L.o,
                                           B, Hk, Hv, dk, dv, dtype);
        for (int m = 0; m < nlayers; ++m) {
            if (m == l) continue;
            const gdn_decode_layer& M = layers[m];
            const DecodeSpans b = decode_spans(M.q, M.k, M.v, M.g, M.beta, M.state_in, M.state_out,
                                               M.o, B, Hk, Hv, dk, dv, dtype);
            for (const Span& out : {a.ss, a.so}) {
                for (const Span& in : b.in)
                    if (overlap(out, in)) return GDN_ERR_ALIAS;
                if (overlap(out, b.ss) || overlap(out, b.so)) return GDN_ERR_ALIAS;
            }
        }
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int l0 = 0; l0 < nlayers; l0 += gdn::kDecodeLayersPerLaunch) {
        gdn::DecodeTable t;
        t.nlayers = nlayers - l0 < gdn::kDecodeLayersPerLaunch ? nlayers - l0 : gdn::kDecodeLayersPerLaunch;
        t.B = B; t.Hk = Hk; t.Hv = Hv; t.qk_norm = (flags & GDN_QK_NORM) ? 1 : 0;
        for (int i = 0; i < gdn::kDecodeLayersPerLaunch; ++i) {
            const gdn_decode_layer& L = layers[l0 + (i < t.nlayers ? i : 0)];
            t.layer[i] = {L.q, L.k, L.v, L.g, L.beta, L.state_in, L.state_out, L.o};
        }
        const hipError_t e = dtype == GDN_BF16 ? gdn::decode_layers_bf16(dk, dv, t, st)
                                               : gdn::decode_layers_f32(dk, dv, t, st);
        if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid sizes (B, T, Hk, Hv) or Hv not a multiple of Hk";
        case GDN_ERR_UNSUPPORTED: return "unsupported dk, dv, chunk or dtype";
        case GDN_ERR_ALIGN: return "misaligned pointer";
        case GDN_ERR_ALIAS: return "an output overlaps another argument";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "HIP runtime error while enqueueing";
    }
    return "unknown status";
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
