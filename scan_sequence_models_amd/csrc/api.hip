// api.hip -- the C ABI declared in include/gdscan.h: argument validation,
// workspace sizing, path selection and error reporting.  No device code here.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdscan.h"
#include "kernels.hpp"
#include "blelloch.hpp"

namespace {

thread_local char g_err[512] = "no error";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};
Range range(const char* name, const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}
bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int hip_fail(hipError_t e, const char* what) {
    return fail(SCAN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Number of compute units of the current device (cached per device).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

struct Plan {
    int path;          // SCAN_PATH_SEQUENTIAL or SCAN_PATH_BLELLOCH
    bool mfma;         // bf16 MFMA kernel (else float32 kernel)
    bool diag;         // diagonal-gate kernel
    int leaf_chunks;   // Blelloch leaf size in chunks
    size_t workspace;  // bytes
};

bool valid_mode(int mode) {
    return mode == SCAN_GDN || mode == SCAN_GLA || mode == SCAN_GDN_EW || mode == SCAN_GDN_DIAG ||
           mode == SCAN_GLA_DIAG;
}
bool diag_mode(int mode) { return mode == SCAN_GDN_DIAG || mode == SCAN_GLA_DIAG; }
bool gla_mode(int mode) { return mode == SCAN_GLA || mode == SCAN_GLA_DIAG; }
// Kernel mode: 0 = gated delta rule (erase and write strengths may differ), 1 = GLA.
int kernel_mode(int mode) { return gla_mode(mode) ? 1 : 0; }
// Elements of the beta argument per token: 1, none (GLA), or 2 planes (split strengths).
int beta_planes(int mode) { return gla_mode(mode) ? 0 : mode == SCAN_GDN_EW ? 2 : 1; }

// Validates the sizes/enums of a scan_fwd call and picks the kernels.
int plan_scan(int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk,
              const scan_opts* opts, Plan* plan) {
    if (!valid_mode(mode))
        return fail(SCAN_EINVAL, "mode must be SCAN_GDN, SCAN_GLA, SCAN_GDN_EW, SCAN_GDN_DIAG or SCAN_GLA_DIAG (got %d)", mode);
    const int km = kernel_mode(mode);
    if (dtype != SCAN_F32 && dtype != SCAN_BF16) return fail(SCAN_EINVAL, "dtype must be SCAN_F32 or SCAN_BF16 (got %d)", dtype);
    if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1)
        return fail(SCAN_EINVAL, "B, H, T, dk, dv must be >= 1 (got %d, %d, %d, %d, %d)", B, H, T, dk, dv);
    if ((int64_t)B * H > INT32_MAX / 64) return fail(SCAN_EINVAL, "B*H too large");
    if (chunk != 16 && chunk != 32 && chunk != 64) return fail(SCAN_EUNSUPPORTED, "chunk must be 16, 32 or 64 (got %d)", chunk);
    const int path = opts ? opts->path : SCAN_PATH_AUTO;
    if (path != SCAN_PATH_AUTO && path != SCAN_PATH_SEQUENTIAL && path != SCAN_PATH_BLELLOCH)
        return fail(SCAN_EINVAL, "opts->path must be SCAN_PATH_AUTO, _SEQUENTIAL or _BLELLOCH (got %d)", path);
    int leaf = opts ? opts->leaf_chunks : 0;
    if (leaf < 0 || (leaf & (leaf - 1)) != 0) return fail(SCAN_EINVAL, "opts->leaf_chunks must be 0 or a power of two (got %d)", leaf);

    Plan p{};
    if (diag_mode(mode)) {  // float32 chunk kernel with per-channel gates, sequential path only
        if (!gds::chunk_diag_supported(dk, dv))
            return fail(SCAN_EUNSUPPORTED, "diagonal gates support dk in {16,32,64,128} and dv a multiple of 16 (got dk=%d dv=%d)", dk, dv);
        if (path == SCAN_PATH_BLELLOCH) return fail(SCAN_EUNSUPPORTED, "diagonal gates run on the sequential path only");
        p.diag = true;
        p.path = SCAN_PATH_SEQUENTIAL;
        *plan = p;
        return SCAN_OK;
    }
    p.mfma = dtype == SCAN_BF16 && gds::chunk_mfma_supported(km, dk, dv, chunk);
    if (!p.mfma && !gds::chunk_f32_supported(km, dk, dv, chunk))
        return fail(SCAN_EUNSUPPORTED, "unsupported size: dk=%d dv=%d chunk=%d (dk in {16,32,64,128}, dv a multiple of 16)", dk, dv, chunk);

    const int64_t nchunks = (T + chunk - 1) / chunk;
    const int64_t heads = (int64_t)B * H;
    p.path = SCAN_PATH_SEQUENTIAL;
    if (path == SCAN_PATH_BLELLOCH) {
        p.path = SCAN_PATH_BLELLOCH;
    } else if (path == SCAN_PATH_AUTO) {
        // The sequential pass runs one workgroup per (head, value slice); when
        // that cannot fill the GPU, split the sequence into leaves and combine
        // their aggregates with the Blelloch tree.  With the delta rule the tree
        // costs about three times the chunk work, so it pays when the
        // sequential grid fills at most a quarter of the CUs (at least two
        // leaves of 16 chunks), or half of them on long sequences; gated linear
        // attention (E = gamma I: no E rows, no dense sweeps) costs about twice
        // the chunk work and pays whenever the grid fills at most half of them.
        const int64_t wgs = heads * gds::sequential_workgroups_per_head(p.mfma, dv);
        const int cus = device_cus();
        const bool gla = km == 1;
        if (gds::blelloch_supported(km, dtype, dk, dv, chunk) &&
            ((wgs * 4 <= cus && nchunks >= 32) || (wgs * 2 <= cus && (nchunks >= 256 || (gla && nchunks >= 32)))))
            p.path = SCAN_PATH_BLELLOCH;
    }
    if (p.path == SCAN_PATH_BLELLOCH) {
        if (!gds::blelloch_supported(km, dtype, dk, dv, chunk))
            return fail(SCAN_EUNSUPPORTED, "the Blelloch path supports dk = dv = 128 only (got dk=%d dv=%d)", dk, dv);
        if (leaf == 0) leaf = gds::blelloch_default_leaf_chunks(nchunks, heads, device_cus());
        p.leaf_chunks = leaf;
        p.workspace = gds::blelloch_workspace_bytes(heads, nchunks, leaf, dk, dv);
    }
    *plan = p;
    return SCAN_OK;
}

// The rest of scan_fwd once the plan is made: pointer checks, then the launch.
int scan_fwd_planned(const Plan& p, int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk,
                     const void* q, const void* k, const void* v, const float* alpha,
                     const float* beta, const float* S0, void* o, float* ST, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !alpha || !o) return fail(SCAN_EINVAL, "q, k, v, alpha and o must be non-null");
    if (!gla_mode(mode) && !beta) return fail(SCAN_EINVAL, "the gated-delta modes need beta");
    if (gla_mode(mode) && beta) return fail(SCAN_EINVAL, "the GLA modes take no beta (pass NULL)");
    const void* a16[] = {q, k, v, o, S0, ST};
    const char* n16[] = {"q", "k", "v", "o", "S0", "ST"};
    for (int i = 0; i < 6; ++i)
        if (a16[i] && !aligned(a16[i], 16)) return fail(SCAN_EALIGN, "%s is not 16-byte aligned", n16[i]);
    if (!aligned(alpha, diag_mode(mode) ? 16 : 4) || (beta && !aligned(beta, 4)))
        return fail(SCAN_EALIGN, "alpha/beta not aligned (alpha 16 bytes with diagonal gates, else 4)");
    if (p.workspace > 0) {
        if (!workspace || workspace_bytes < p.workspace)
            return fail(SCAN_EWORKSPACE, "workspace of %zu bytes required (got %zu)", p.workspace, workspace_bytes);
        if (!aligned(workspace, 256)) return fail(SCAN_EALIGN, "workspace is not 256-byte aligned");
    }
    const size_t es = dtype == SCAN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H;
    const Range in[] = {range("q", q, BH * T * dk * es), range("k", k, BH * T * dk * es),
                        range("v", v, BH * T * dv * es),
                        range("alpha", alpha, BH * T * 4 * (diag_mode(mode) ? dk : 1)),
                        range("beta", beta, BH * T * 4 * beta_planes(mode)),
                        range("S0", S0, BH * dv * dk * 4),
                        range("workspace", workspace, p.workspace)};
    const Range ro = range("o", o, BH * T * dv * es);
    const Range rs = range("ST", ST, BH * dv * dk * 4);
    for (const Range& r : in) {
        if (overlaps(ro, r)) return fail(SCAN_EINVAL, "o overlaps %s", r.name);
        if (overlaps(rs, r) && !(r.name[0] == 'S' && ST == S0))
            return fail(SCAN_EINVAL, "ST overlaps %s (only ST == S0 is allowed)", r.name);
    }
    if (overlaps(ro, rs)) return fail(SCAN_EINVAL, "o overlaps ST");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int km = kernel_mode(mode);
    // split strengths: the write plane follows the erase plane
    const float* beta_w = mode == SCAN_GDN_EW ? beta + BH * T : beta;
    hipError_t e;
    if (p.diag) {
        e = gds::launch_chunk_diag(km, dtype, (int)BH, T, dk, dv, q, k, v, alpha, beta, S0, o, ST, s);
    } else if (p.path == SCAN_PATH_BLELLOCH) {
        e = gds::launch_blelloch(km, (int)BH, T, dk, dv, chunk, p.leaf_chunks, q, k, v, alpha, beta,
                                 beta_w, S0, o, ST, workspace, s);
    } else if (p.mfma) {
        e = gds::launch_chunk_mfma(km, (int)BH, T, dk, dv, chunk, q, k, v, alpha, beta, beta_w, S0, o,
                                   ST, s);
    } else {
        e = gds::launch_chunk_f32(km, dtype, (int)BH, T, dk, dv, chunk, q, k, v, alpha, beta, beta_w,
                                  S0, o, ST, s);
    }
    if (e != hipSuccess) return hip_fail(e, "scan_fwd launch");
    return SCAN_OK;
}

}  // namespace

extern "C" {

const char* scan_last_error(void) { return g_err; }

const char* scan_version(void) { return "gdscan 0.1.0 (gfx950, HIP)"; }

size_t scan_fwd_workspace_size(int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk,
                               const scan_opts* opts) {
    Plan p;
    if (plan_scan(mode, dtype, B, H, T, dk, dv, chunk, opts, &p) != SCAN_OK) return (size_t)-1;
    return p.workspace;
}

int scan_fwd(int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk, const void* q,
             const void* k, const void* v, const float* alpha, const float* beta, const float* S0,
             void* o, float* ST, void* workspace, size_t workspace_bytes, const scan_opts* opts,
             void* stream) {
    Plan p;
    const int st = plan_scan(mode, dtype, B, H, T, dk, dv, chunk, opts, &p);
    if (st != SCAN_OK) return st;
    return scan_fwd_planned(p, mode, dtype, B, H, T, dk, dv, chunk, q, k, v, alpha, beta, S0, o, ST,
                            workspace, workspace_bytes, stream);
}

int scan_fwd_noalloc(int mode, int dtype, int B, int H, int T, int dk, int dv, int chunk,
                     const void* q, const void* k, const void* v, const float* alpha,
                     const float* beta, const float* S0, void* o, float* ST,
                     const scan_opts* opts, void* stream) {
    Plan p;
    const int st = plan_scan(mode, dtype, B, H, T, dk, dv, chunk, opts, &p);
    if (st != SCAN_OK) return st;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (p.workspace > 0) {
        if (p.workspace > (size_t)SCAN_NOALLOC_MAX_WORKSPACE)
            return fail(SCAN_EWORKSPACE,
                        "scan_fwd_noalloc: these arguments need %zu bytes of scratch, above the fixed "
                        "%zu bytes it has (use scan_fwd with a caller workspace)",
                        p.workspace, (size_t)SCAN_NOALLOC_MAX_WORKSPACE);
        const hipError_t e = gds::noalloc_scratch(&ws);
        if (e != hipSuccess) return hip_fail(e, "scan_fwd_noalloc: address of the device scratch");
        ws_bytes = SCAN_NOALLOC_MAX_WORKSPACE;
    }
    return scan_fwd_planned(p, mode, dtype, B, H, T, dk, dv, chunk, q, k, v, alpha, beta, S0, o, ST, ws,
                            ws_bytes, stream);
}

int decode_step(int mode, int dtype, int N, int dk, int dv, const void* q, const void* k,
                const void* v, const float* alpha, const float* beta, float* S, void* o,
                void* stream) {
    if (!valid_mode(mode))
        return fail(SCAN_EINVAL, "mode must be SCAN_GDN, SCAN_GLA, SCAN_GDN_EW, SCAN_GDN_DIAG or SCAN_GLA_DIAG (got %d)", mode);
    if (dtype != SCAN_F32 && dtype != SCAN_BF16) return fail(SCAN_EINVAL, "dtype must be SCAN_F32 or SCAN_BF16 (got %d)", dtype);
    if (N < 1 || dk < 1 || dv < 1) return fail(SCAN_EINVAL, "N, dk, dv must be >= 1 (got %d, %d, %d)", N, dk, dv);
    if (!gds::decode_supported(dk)) return fail(SCAN_EUNSUPPORTED, "decode_step supports dk in {16,32,64,128} (got %d)", dk);
    if ((int64_t)N * ((dv + 31) / 32) > INT32_MAX) return fail(SCAN_EINVAL, "N*dv too large");  // one workgroup per 32 rows
    if (!q || !k || !v || !alpha || !S || !o) return fail(SCAN_EINVAL, "q, k, v, alpha, S and o must be non-null");
    if (!gla_mode(mode) && !beta) return fail(SCAN_EINVAL, "the gated-delta modes need beta");
    if (gla_mode(mode) && beta) return fail(SCAN_EINVAL, "the GLA modes take no beta (pass NULL)");
    const void* a16[] = {q, k, v, o, S};
    const char* n16[] = {"q", "k", "v", "o", "S"};
    for (int i = 0; i < 5; ++i)
        if (!aligned(a16[i], 16)) return fail(SCAN_EALIGN, "%s is not 16-byte aligned", n16[i]);
    if (!aligned(alpha, diag_mode(mode) ? 16 : 4) || (beta && !aligned(beta, 4)))
        return fail(SCAN_EALIGN, "alpha/beta not aligned (alpha 16 bytes with diagonal gates, else 4)");
    const size_t es = dtype == SCAN_BF16 ? 2 : 4;
    const Range in[] = {range("q", q, (size_t)N * dk * es), range("k", k, (size_t)N * dk * es),
                        range("v", v, (size_t)N * dv * es),
                        range("alpha", alpha, (size_t)N * 4 * (diag_mode(mode) ? dk : 1)),
                        range("beta", beta, (size_t)N * 4 * beta_planes(mode)),
                        range("S", S, (size_t)N * dv * dk * 4)};
    const Range ro = range("o", o, (size_t)N * dv * es);
    for (const Range& r : in)
        if (overlaps(ro, r)) return fail(SCAN_EINVAL, "o overlaps %s", r.name);
    const Range rS = in[5];
    for (int i = 0; i < 5; ++i)
        if (overlaps(rS, in[i])) return fail(SCAN_EINVAL, "S overlaps %s", in[i].name);
    const float* beta_w = mode == SCAN_GDN_EW ? beta + N : beta;
    const int dmode = kernel_mode(mode) + (diag_mode(mode) ? 2 : 0);
    hipError_t e = gds::launch_decode(dmode, dtype, N, dk, dv, q, k, v, alpha, beta, beta_w, S, o,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode_step launch");
    return SCAN_OK;
}

int prism_expand(int dtype, int B, int H, int T, int dk, int dv, int L, int W, const void* q,
                 const void* k, const void* v, const void* x, const float* alpha, const float* beta,
                 const float* beta_l, const float* conv, const void* Wk, const void* Wp, void* q2,
                 void* k2, void* v2, float* alpha2, float* beta2, void* stream) {
    if (dtype != SCAN_F32 && dtype != SCAN_BF16) return fail(SCAN_EINVAL, "dtype must be SCAN_F32 or SCAN_BF16 (got %d)", dtype);
    if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1)
        return fail(SCAN_EINVAL, "B, H, T, dk, dv must be >= 1 (got %d, %d, %d, %d, %d)", B, H, T, dk, dv);
    if (L < 0 || L > PRISM_MAX_STEPS) return fail(SCAN_EINVAL, "L must be in [0, %d] (got %d)", PRISM_MAX_STEPS, L);
    if (W < 1 || W > PRISM_MAX_WINDOW) return fail(SCAN_EINVAL, "W must be in [1, %d] (got %d)", PRISM_MAX_WINDOW, W);
    if (!gds::prism_supported(dtype, dk, dv))
        return fail(SCAN_EUNSUPPORTED, "prism_expand supports dk, dv in {16, 32, 64, 128} (got %d, %d)", dk, dv);
    const int64_t G = L + 1;
    if ((int64_t)T * G > INT32_MAX / 2 || (int64_t)B * H > INT32_MAX / 64 ||
        (int64_t)B * H * ((T + 15) / 16) > INT32_MAX)
        return fail(SCAN_EINVAL, "B*H and T*(L+1) too large");
    if (!q || !k || !v || !alpha || !beta || !q2 || !k2 || !v2 || !alpha2 || !beta2)
        return fail(SCAN_EINVAL, "q, k, v, alpha, beta and the five outputs must be non-null");
    if (L > 0 && (!x || !beta_l || !conv || !Wk || !Wp))
        return fail(SCAN_EINVAL, "L > 0 needs x, beta_l, conv, Wk and Wp");
    const void* a16[] = {q, k, v, x, conv, Wk, Wp, q2, k2, v2};
    const char* n16[] = {"q", "k", "v", "x", "conv", "Wk", "Wp", "q2", "k2", "v2"};
    for (int i = 0; i < 10; ++i)
        if (a16[i] && !aligned(a16[i], 16)) return fail(SCAN_EALIGN, "%s is not 16-byte aligned", n16[i]);
    const void* a4[] = {alpha, beta, beta_l, alpha2, beta2};
    for (const void* p : a4)
        if (p && !aligned(p, 4)) return fail(SCAN_EALIGN, "gate arrays must be 4-byte aligned");
    const size_t es = dtype == SCAN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H, T2 = (size_t)T * G;
    const Range in[] = {range("q", q, BH * T * dk * es), range("k", k, BH * T * dk * es),
                        range("v", v, BH * T * dv * es), range("x", x, L ? BH * T * dv * es : 0),
                        range("alpha", alpha, BH * T * 4), range("beta", beta, BH * T * 4),
                        range("beta_l", beta_l, BH * T * L * 4),
                        range("conv", conv, L ? (size_t)H * W * dv * 4 : 0),
                        range("Wk", Wk, (size_t)H * L * dk * dv * es),
                        range("Wp", Wp, (size_t)H * L * dv * dv * es)};
    const Range out[] = {range("q2", q2, BH * T2 * dk * es), range("k2", k2, BH * T2 * dk * es),
                         range("v2", v2, BH * T2 * dv * es), range("alpha2", alpha2, BH * T2 * 4),
                         range("beta2", beta2, 2 * BH * T2 * 4)};
    for (int a = 0; a < 5; ++a) {
        for (const Range& r : in)
            if (overlaps(out[a], r)) return fail(SCAN_EINVAL, "%s overlaps %s", out[a].name, r.name);
        for (int b = a + 1; b < 5; ++b)
            if (overlaps(out[a], out[b])) return fail(SCAN_EINVAL, "%s overlaps %s", out[a].name, out[b].name);
    }
    gds::PrismJob j{};
    j.q = q; j.k = k; j.v = v; j.x = x;
    j.alpha = alpha; j.beta = beta; j.beta_l = beta_l; j.conv = conv;
    j.Wk = Wk; j.Wp = Wp;
    j.q2 = q2; j.k2 = k2; j.v2 = v2; j.alpha2 = alpha2; j.beta2 = beta2;
    j.BH = (int)BH; j.H = H; j.T = T; j.dk = dk; j.dv = dv; j.L = L; j.W = W;
    hipError_t e = gds::launch_prism_expand(dtype, j, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prism_expand launch");
    return SCAN_OK;
}

namespace {
// Validates the sizes of a prism_scan call; returns SCAN_OK and the workspace bytes.
int plan_prism_scan(int dtype, int B, int H, int T, int dk, int dv, int L, size_t* ws) {
    if (dtype != SCAN_BF16) return fail(SCAN_EUNSUPPORTED, "prism_scan runs on bfloat16 data (dtype SCAN_BF16)");
    if (B < 1 || H < 1 || T < 1) return fail(SCAN_EINVAL, "B, H, T must be >= 1 (got %d, %d, %d)", B, H, T);
    if (dk != 128 || dv != 128) return fail(SCAN_EUNSUPPORTED, "prism_scan supports dk = dv = 128 (got %d, %d)", dk, dv);
    if (L < 0 || L > PRISM_MAX_STEPS) return fail(SCAN_EINVAL, "L must be in [0, %d] (got %d)", PRISM_MAX_STEPS, L);
    if ((int64_t)B * H > INT32_MAX / 64) return fail(SCAN_EINVAL, "B*H too large");
    if (L > 0 && !gds::chunk_prism_supported(T, L))
        return fail(SCAN_EUNSUPPORTED, "T (L + 1) = %lld elements is too long for prism_scan", (long long)T * (L + 1));
    *ws = (size_t)B * H * T * L * (dk + dv) * 2;
    return SCAN_OK;
}
}  // namespace

size_t prism_scan_workspace_size(int dtype, int B, int H, int T, int dk, int dv, int L) {
    size_t ws = 0;
    if (plan_prism_scan(dtype, B, H, T, dk, dv, L, &ws) != SCAN_OK) return (size_t)-1;
    return ws;
}

int prism_scan(int dtype, int B, int H, int T, int dk, int dv, int L, int W, const void* q,
               const void* k, const void* v, const void* x, const float* alpha, const float* beta,
               const float* beta_l, const float* conv, const void* Wk, const void* Wp,
               const float* S0, void* o, float* ST, void* workspace, size_t workspace_bytes,
               void* stream) {
    size_t need = 0;
    int st = plan_prism_scan(dtype, B, H, T, dk, dv, L, &need);
    if (st != SCAN_OK) return st;
    if (W < 1 || W > PRISM_MAX_WINDOW) return fail(SCAN_EINVAL, "W must be in [1, %d] (got %d)", PRISM_MAX_WINDOW, W);
    if (!q || !k || !v || !alpha || !beta || !o) return fail(SCAN_EINVAL, "q, k, v, alpha, beta and o must be non-null");
    if (L > 0 && (!x || !beta_l || !conv || !Wk || !Wp))
        return fail(SCAN_EINVAL, "L > 0 needs x, beta_l, conv, Wk and Wp");
    const void* a16[] = {q, k, v, x, conv, Wk, Wp, S0, o, ST};
    const char* n16[] = {"q", "k", "v", "x", "conv", "Wk", "Wp", "S0", "o", "ST"};
    for (int i = 0; i < 10; ++i)
        if (a16[i] && !aligned(a16[i], 16)) return fail(SCAN_EALIGN, "%s is not 16-byte aligned", n16[i]);
    const void* a4[] = {alpha, beta, beta_l};
    for (const void* p : a4)
        if (p && !aligned(p, 4)) return fail(SCAN_EALIGN, "gate arrays must be 4-byte aligned");
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(SCAN_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
        if (!aligned(workspace, 256)) return fail(SCAN_EALIGN, "workspace is not 256-byte aligned");
    }
    const size_t BH = (size_t)B * H;
    const size_t es = 2;
    const Range in[] = {range("q", q, BH * T * dk * es), range("k", k, BH * T * dk * es),
                        range("v", v, BH * T * dv * es), range("x", x, L ? BH * T * dv * es : 0),
                        range("alpha", alpha, BH * T * 4), range("beta", beta, BH * T * 4),
                        range("beta_l", beta_l, BH * T * L * 4),
                        range("conv", conv, L ? (size_t)H * W * dv * 4 : 0),
                        range("Wk", Wk, (size_t)H * L * dk * dv * es),
                        range("Wp", Wp, (size_t)H * L * dv * dv * es),
                        range("S0", S0, BH * dv * dk * 4),
                        range("workspace", workspace, need)};
    const Range ro = range("o", o, BH * T * dv * es);
    const Range rs = range("ST", ST, BH * dv * dk * 4);
    for (const Range& r : in) {
        if (overlaps(ro, r)) return fail(SCAN_EINVAL, "o overlaps %s", r.name);
        if (overlaps(rs, r) && !(r.name[0] == 'S' && ST == S0))
            return fail(SCAN_EINVAL, "ST overlaps %s (only ST == S0 is allowed)", r.name);
    }
    if (overlaps(ro, rs)) return fail(SCAN_EINVAL, "o overlaps ST");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (L == 0) {  // no corrections: the gated-delta scan itself
        e = gds::launch_chunk_mfma(0, (int)BH, T, dk, dv, 64, q, k, v, alpha, beta, beta, S0, o, ST, s);
        if (e != hipSuccess) return hip_fail(e, "prism_scan launch");
        return SCAN_OK;
    }
    gds::PrismJob j{};
    j.q = q; j.k = k; j.v = v; j.x = x;
    j.alpha = alpha; j.beta = beta; j.beta_l = beta_l; j.conv = conv;
    j.Wk = Wk; j.Wp = Wp;
    j.kf = workspace;
    j.vf = static_cast<char*>(workspace) + BH * T * L * dk * es;
    j.BH = (int)BH; j.H = H; j.T = T; j.dk = dk; j.dv = dv; j.L = L; j.W = W;
    e = gds::launch_prism_factors(j, s);
    if (e == hipSuccess)
        e = gds::launch_chunk_prism((int)BH, T, L, q, k, v, j.kf, j.vf, alpha, beta, beta_l, S0, o, ST, s);
    if (e != hipSuccess) return hip_fail(e, "prism_scan launch");
    return SCAN_OK;
}

namespace {
// Validates the sizes of a lact_fwd call; returns SCAN_OK and the workspace bytes.
int plan_lact(int dtype, int B, int H, int T, int dk, int dv, int chunk, size_t* ws) {
    if (dtype != SCAN_F32 && dtype != SCAN_BF16) return fail(SCAN_EINVAL, "dtype must be SCAN_F32 or SCAN_BF16 (got %d)", dtype);
    if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1 || chunk < 1)
        return fail(SCAN_EINVAL, "B, H, T, dk, dv, chunk must be >= 1 (got %d, %d, %d, %d, %d, %d)", B, H, T, dk, dv, chunk);
    if ((int64_t)B * H > INT32_MAX / 64 || (int64_t)B * H * ((T + 63) / 64) > INT32_MAX)
        return fail(SCAN_EINVAL, "B*H*T too large");
    if (gds::lact_mfma_supported(dtype, dk, dv, chunk)) {
        *ws = gds::lact_workspace_bytes((int64_t)B * H, T, chunk);
        return SCAN_OK;
    }
    if (gds::lact_plain_supported(dk, dv)) {
        *ws = 0;
        return SCAN_OK;
    }
    return fail(SCAN_EUNSUPPORTED,
                "lact_fwd supports bf16 with dk = dv = 128 and chunk a multiple of 64, or dk, dv in {16, 32, 64} "
                "(got dtype %d, dk %d, dv %d, chunk %d)", dtype, dk, dv, chunk);
}
}  // namespace

size_t lact_fwd_workspace_size(int dtype, int B, int H, int T, int dk, int dv, int chunk) {
    size_t ws = 0;
    if (plan_lact(dtype, B, H, T, dk, dv, chunk, &ws) != SCAN_OK) return (size_t)-1;
    return ws;
}

int lact_fwd(int dtype, int B, int H, int T, int dk, int dv, int chunk, int order, const void* q,
             const void* k, const void* v, const float* eta, const float* W0, void* o, float* WT,
             void* workspace, size_t workspace_bytes, void* stream) {
    size_t need = 0;
    int st = plan_lact(dtype, B, H, T, dk, dv, chunk, &need);
    if (st != SCAN_OK) return st;
    if (order != LACT_UPDATE_THEN_APPLY && order != LACT_APPLY_THEN_UPDATE)
        return fail(SCAN_EINVAL, "order must be LACT_UPDATE_THEN_APPLY or LACT_APPLY_THEN_UPDATE (got %d)", order);
    if (!q || !k || !v || !eta || !o) return fail(SCAN_EINVAL, "q, k, v, eta and o must be non-null");
    const void* a16[] = {q, k, v, o, W0, WT};
    const char* n16[] = {"q", "k", "v", "o", "W0", "WT"};
    for (int i = 0; i < 6; ++i)
        if (a16[i] && !aligned(a16[i], 16)) return fail(SCAN_EALIGN, "%s is not 16-byte aligned", n16[i]);
    if (!aligned(eta, 4)) return fail(SCAN_EALIGN, "eta is not 4-byte aligned");
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(SCAN_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
        if (!aligned(workspace, 256)) return fail(SCAN_EALIGN, "workspace is not 256-byte aligned");
    }
    const size_t es = dtype == SCAN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H;
    const Range in[] = {range("q", q, BH * T * dk * es), range("k", k, BH * T * dk * es),
                        range("v", v, BH * T * dv * es), range("eta", eta, BH * T * 4),
                        range("W0", W0, BH * dv * dk * 4), range("workspace", workspace, need)};
    const Range ro = range("o", o, BH * T * dv * es);
    const Range rw = range("WT", WT, BH * dv * dk * 4);
    for (const Range& r : in) {
        if (overlaps(ro, r)) return fail(SCAN_EINVAL, "o overlaps %s", r.name);
        if (overlaps(rw, r) && !(r.name[0] == 'W' && WT == W0))
            return fail(SCAN_EINVAL, "WT overlaps %s (only WT == W0 is allowed)", r.name);
    }
    if (overlaps(ro, rw)) return fail(SCAN_EINVAL, "o overlaps WT");
    gds::LactJob j{};
    j.q = q; j.k = k; j.v = v; j.eta = eta; j.W0 = W0; j.o = o; j.WT = WT;
    j.BH = (int)BH; j.T = T; j.dk = dk; j.dv = dv; j.chunk = chunk; j.order = order;
    hipError_t e = gds::launch_lact(dtype, j, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lact_fwd launch");
    return SCAN_OK;
}

namespace {
// Validates the sizes of a scan_bwd call; returns SCAN_OK and the workspace bytes.
int plan_bwd(int mode, int dtype, int B, int H, int T, int dk, int dv, size_t* ws) {
    if (mode != SCAN_GDN && mode != SCAN_GLA && mode != SCAN_GDN_EW)
        return fail(SCAN_EUNSUPPORTED, "scan_bwd supports SCAN_GDN, SCAN_GLA and SCAN_GDN_EW (got mode %d)", mode);
    if (dtype != SCAN_F32 && dtype != SCAN_BF16) return fail(SCAN_EINVAL, "dtype must be SCAN_F32 or SCAN_BF16 (got %d)", dtype);
    if (B < 1 || H < 1 || T < 1 || dk < 1 || dv < 1)
        return fail(SCAN_EINVAL, "B, H, T, dk, dv must be >= 1 (got %d, %d, %d, %d, %d)", B, H, T, dk, dv);
    if ((int64_t)B * H * (dv / 64 + 1) > INT32_MAX / 2 || (int64_t)B * H * T > INT32_MAX)
        return fail(SCAN_EINVAL, "B*H*T too large");
    if (!gds::scan_bwd_supported(dk, dv))
        return fail(SCAN_EUNSUPPORTED, "scan_bwd supports dk in {32, 64, 128} and dv a multiple of 64 up to 4096 "
                    "(got dk %d, dv %d)", dk, dv);
    *ws = gds::scan_bwd_workspace_floats(B * H, T, dk, dv) * sizeof(float);
    return SCAN_OK;
}
}  // namespace

size_t scan_bwd_workspace_size(int mode, int dtype, int B, int H, int T, int dk, int dv) {
    size_t ws = 0;
    if (plan_bwd(mode, dtype, B, H, T, dk, dv, &ws) != SCAN_OK) return (size_t)-1;
    return ws;
}

int scan_bwd(int mode, int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
             const void* v, const float* alpha, const float* beta, const float* S0, const void* dO,
             const float* dST, float* dq, float* dk_out, float* dv_out, float* dalpha, float* dbeta,
             float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
    size_t need = 0;
    int st = plan_bwd(mode, dtype, B, H, T, dk, dv, &need);
    if (st != SCAN_OK) return st;
    const bool gdn = mode != SCAN_GLA;
    const size_t planes = mode == SCAN_GDN_EW ? 2 : 1;
    if (!q || !k || !v || !alpha || !dq || !dk_out || !dv_out || !dalpha || !dS0)
        return fail(SCAN_EINVAL, "q, k, v, alpha, dq, dk, dv, dalpha and dS0 must be non-null");
    if (gdn && (!beta || !dbeta)) return fail(SCAN_EINVAL, "the delta rule needs beta and dbeta");
    if (!gdn && (beta || dbeta)) return fail(SCAN_EINVAL, "SCAN_GLA takes no beta and no dbeta (pass NULL)");
    const void* a16[] = {q, k, v, dO, S0, dST, dq, dk_out, dv_out, dS0};
    const char* n16[] = {"q", "k", "v", "dO", "S0", "dST", "dq", "dk", "dv", "dS0"};
    for (int i = 0; i < 10; ++i)
        if (a16[i] && !aligned(a16[i], 16)) return fail(SCAN_EALIGN, "%s is not 16-byte aligned", n16[i]);
    const void* a4[] = {alpha, beta, dalpha, dbeta};
    for (const void* p : a4)
        if (p && !aligned(p, 4)) return fail(SCAN_EALIGN, "alpha, beta, dalpha, dbeta must be 4-byte aligned");
    if (!workspace || workspace_bytes < need)
        return fail(SCAN_EWORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (!aligned(workspace, 256)) return fail(SCAN_EALIGN, "workspace is not 256-byte aligned");
    const size_t es = dtype == SCAN_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H;
    const Range in[] = {range("q", q, BH * T * dk * es), range("k", k, BH * T * dk * es),
                        range("v", v, BH * T * dv * es), range("alpha", alpha, BH * T * 4),
                        range("beta", beta, planes * BH * T * 4), range("S0", S0, BH * dv * dk * 4),
                        range("dO", dO, BH * T * dv * es), range("dST", dST, BH * dv * dk * 4)};
    const Range out[] = {range("dq", dq, BH * T * dk * 4), range("dk", dk_out, BH * T * dk * 4),
                         range("dv", dv_out, BH * T * dv * 4), range("dalpha", dalpha, BH * T * 4),
                         range("dbeta", dbeta, planes * BH * T * 4), range("dS0", dS0, BH * dv * dk * 4),
                         range("workspace", workspace, need)};
    for (size_t a = 0; a < sizeof(out) / sizeof(out[0]); ++a) {
        for (const Range& r : in)
            if (overlaps(out[a], r)) return fail(SCAN_EINVAL, "%s overlaps %s", out[a].name, r.name);
        for (size_t b = a + 1; b < sizeof(out) / sizeof(out[0]); ++b)
            if (overlaps(out[a], out[b])) return fail(SCAN_EINVAL, "%s overlaps %s", out[a].name, out[b].name);
    }
    gds::BwdJob j{};
    j.q = q; j.k = k; j.v = v; j.dO = dO;
    j.alpha = alpha; j.beta = beta; j.S0 = S0; j.dST = dST;
    j.beta_w = planes == 2 ? beta + BH * T : beta;
    j.dq = dq; j.dk_out = dk_out; j.dv_out = dv_out; j.dalpha = dalpha; j.dbeta = dbeta; j.dS0 = dS0;
    j.dbeta_w = planes == 2 ? dbeta + BH * T : nullptr;
    j.ckpt = static_cast<float*>(workspace);
    j.BH = (int)BH; j.T = T; j.dk = dk; j.dv = dv;
    hipError_t e = gds::launch_scan_bwd(gdn ? 0 : 1, dtype == SCAN_BF16 ? 1 : 0, j, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "scan_bwd launch");
    return SCAN_OK;
}

}  // extern "C"
