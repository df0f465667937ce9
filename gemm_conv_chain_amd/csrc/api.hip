// api.hip -- the C ABI of libfusedchain (declared in include/fusedchain.h):
// host-side argument validation, variant choice and launch on the caller's
// stream.  Validation happens before any HIP call.
#include <stdarg.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <tuple>

#include "../../include/fusedchain.h"
#include "fc_launch.h"

namespace fc {
hipError_t run_conv_bias_act3x3(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act,
                                half_t* y, int NB, int H, int W, int C, int K, hipStream_t st);
hipError_t run_conv_pool3x3(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act,
                            bool avg, half_t* y, uint8_t* argmax, int NB, int H, int W, int C, int K, bool regw,
                            hipStream_t st);
bool conv_pool_wr_fits(int W, int C, int K);
hipError_t run_chain_conv2_3x3(const half_t* x, const half_t* w0, const half_t* b0, int act, const half_t* w1,
                               const half_t* b1, half_t* y, int NB, int H, int W, int C, int K0, int K1,
                               hipStream_t st);
hipError_t run_chain_convN_3x3(const half_t* x, int nst, const half_t* const* w, const half_t* const* b,
                               const int* act, const int* widths, half_t* y, int NB, int H, int W, int C,
                               hipStream_t st);
bool gemmn_fits(int nst, const int* widths);
hipError_t run_pool2x2(bool avg, const half_t* v, half_t* y, uint8_t* am, int NB, int P, int Q, int K,
                       hipStream_t st);
hipError_t run_pad_mid(const half_t* src, half_t* dst, long outer, int c_in, int c_out, int inner, hipStream_t st);
bool convw_fits(int C, int K);
}  // namespace fc

using fc::half_t;

namespace {

thread_local char g_err[256];

fc_status fail(fc_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

fc_status ok()
{
    g_err[0] = 0;
    return FC_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

fc_status hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(FC_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

const half_t* H(const fc_half* p) { return reinterpret_cast<const half_t*>(p); }
half_t* Hm(fc_half* p) { return reinterpret_cast<half_t*>(p); }

fc_status check_act(fc_act act)
{
    if ((int)act < 0 || (int)act > 3) return fail(FC_E_ARG, "act %d out of range", (int)act);
    return FC_OK;
}

// Shapes the conv kernels implement: 3x3, stride 1, pad 1, c % 32, k % 8.
fc_status check_conv(const fc_conv_shape* s, int kmax)
{
    if (!s) return fail(FC_E_NULL, "shape is NULL");
    if (s->n < 0 || s->h < 0 || s->w < 0 || s->c <= 0 || s->k <= 0 || s->r <= 0 || s->s <= 0 || s->stride <= 0 ||
        s->pad < 0)
        return fail(FC_E_SHAPE, "bad conv shape");
    if (s->c % 8 || s->k % 8) return fail(FC_E_SHAPE, "c=%d and k=%d must be multiples of 8", s->c, s->k);
    if (s->r != 3 || s->s != 3 || s->stride != 1 || s->pad != 1)
        return fail(FC_E_UNSUPPORTED, "only 3x3 stride-1 pad-1 convolutions are implemented");
    if (s->c % 32) return fail(FC_E_UNSUPPORTED, "c=%d: pad channels to a multiple of 32", s->c);
    if (s->k > kmax) return fail(FC_E_UNSUPPORTED, "k=%d exceeds the %d output channels one block keeps", s->k, kmax);
    if ((long)s->n * s->h * s->w > 0x7fffffffL)
        return fail(FC_E_UNSUPPORTED, "n*h*w exceeds 2^31 - 1 pixels (pixel indices are 32-bit)");
    // tap offsets from a pixel (or a pool window's first pixel) to its 3x3
    // neighbours span less than 2 (w + 2) c elements and are 32-bit
    if (((long)s->w + 2) * s->c >= (1L << 30))
        return fail(FC_E_UNSUPPORTED, "(w+2)*c=%ld: 3x3 tap offsets would exceed 32 bits", ((long)s->w + 2) * s->c);
    return FC_OK;
}


// Shape rules of chain_gemm2 (no pointers): residence, multiples of 8, the
// activation, and which variants apply.
fc_status check_g2_shape(int64_t M, int32_t K0, int32_t N0, int32_t N1, fc_act act, bool* rf_ok, bool* stream_ok)
{
    if (M < 0 || K0 <= 0 || N0 <= 0 || N1 <= 0) return fail(FC_E_SHAPE, "M>=0 and K0, N0, N1 > 0 required");
    if (K0 % 8 || N0 % 8 || N1 % 8) return fail(FC_E_SHAPE, "K0, N0, N1 must be multiples of 8");
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    if (N0 > 256) return fail(FC_E_UNSUPPORTED, "N0=%d exceeds the residence limit of 256", N0);
    *rf_ok = N0 <= 128 && fc::rf_fits(K0, N0, N1);
    *stream_ok = fc::stream_fits(N0, N1);
    return FC_OK;
}

fc_status check_g2_ptrs(const fc_half* A, const fc_half* W0, const fc_half* b0, const fc_half* W1, const fc_half* b1,
                        const fc_half* D1, int64_t M)
{
    if (!W0 || !W1 || (M > 0 && (!A || !D1))) return fail(FC_E_NULL, "A, W0, W1 and D1 are required");
    if (!aligned16(A) || !aligned16(W0) || !aligned16(W1) || !aligned16(D1) || !aligned16(b0) || !aligned16(b1))
        return fail(FC_E_ALIGN, "tensor pointers must be 16-byte aligned");
    return FC_OK;
}

// Tuned variant choices (chain_gemm2_tune), per device and shape.
typedef std::tuple<int, int64_t, int32_t, int32_t, int32_t, int> TuneKey;   // device, M, K0, N0, N1, act
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tune;

int rule_variant(bool rf_ok, bool stream_ok)
{
    return rf_ok ? fc::VARIANT_RF : (stream_ok ? fc::VARIANT_STREAM : fc::VARIANT_LDS);
}

// The variant FC_VARIANT_AUTO runs: the tuned one for this device and shape if
// any, else the static rule.  The device is only queried when something has
// been tuned.
int auto_variant(int64_t M, int32_t K0, int32_t N0, int32_t N1, int act, bool rf_ok, bool stream_ok)
{
    {
        std::lock_guard<std::mutex> g(g_tune_mu);
        if (!g_tune.empty()) {
            int dev = 0;
            if (hipGetDevice(&dev) == hipSuccess) {
                auto it = g_tune.find(TuneKey(dev, M, K0, N0, N1, act));
                if (it != g_tune.end()) return it->second;
            }
        }
    }
    return rule_variant(rf_ok, stream_ok);
}

}  // namespace

extern "C" {

int32_t fc_abi_version(void) { return FC_ABI_VERSION; }

const char* fc_status_str(fc_status s)
{
    switch (s) {
    case FC_OK: return "FC_OK";
    case FC_E_NULL: return "FC_E_NULL";
    case FC_E_SHAPE: return "FC_E_SHAPE";
    case FC_E_ALIGN: return "FC_E_ALIGN";
    case FC_E_UNSUPPORTED: return "FC_E_UNSUPPORTED";
    case FC_E_HIP: return "FC_E_HIP";
    case FC_E_ARG: return "FC_E_ARG";
    }
    return "FC_E_UNKNOWN";
}

const char* fc_last_error(void) { return g_err; }

fc_status chain_gemm2_variant(const fc_half* A, const fc_half* W0, const fc_half* b0, fc_act act,
                              const fc_half* W1, const fc_half* b1, fc_half* D1, int64_t M, int32_t K0, int32_t N0,
                              int32_t N1, fc_variant variant, void* stream)
{
    bool rf_ok = false, stream_ok = false;
    if (M < 0 || K0 <= 0 || N0 <= 0 || N1 <= 0) return fail(FC_E_SHAPE, "M>=0 and K0, N0, N1 > 0 required");
    fc_status s = check_g2_ptrs(A, W0, b0, W1, b1, D1, M);
    if (s != FC_OK) return s;
    s = check_g2_shape(M, K0, N0, N1, act, &rf_ok, &stream_ok);
    if (s != FC_OK) return s;
    if ((int)variant < 0 || (int)variant > 3) return fail(FC_E_ARG, "variant %d out of range", (int)variant);
    int v = variant;
    if (v == FC_VARIANT_RF && !rf_ok)
        return fail(FC_E_UNSUPPORTED, "register-resident variant needs N0<=128 and W0,W1 within LDS");
    if (v == FC_VARIANT_STREAM && !stream_ok)
        return fail(FC_E_UNSUPPORTED, "streamed variant needs N1<=16128 (biases beside the weight buffers)");
    if (M == 0) return ok();
    if (v == FC_VARIANT_AUTO) v = auto_variant(M, K0, N0, N1, (int)act, rf_ok, stream_ok);
    return hip_status(fc::run_chain_gemm2(H(A), H(W0), H(b0), act, H(W1), H(b1), Hm(D1), M, K0, N0, N1, v,
                                          (hipStream_t)stream),
                      "chain_gemm2");
}

fc_status chain_gemm2_tune(const fc_half* A, const fc_half* W0, const fc_half* b0, fc_act act, const fc_half* W1,
                           const fc_half* b1, fc_half* D1, int64_t M, int32_t K0, int32_t N0, int32_t N1,
                           int32_t reps, fc_variant* best, float* us, void* stream)
{
    bool rf_ok = false, stream_ok = false;
    if (M < 0 || K0 <= 0 || N0 <= 0 || N1 <= 0) return fail(FC_E_SHAPE, "M>=0 and K0, N0, N1 > 0 required");
    fc_status s = check_g2_ptrs(A, W0, b0, W1, b1, D1, M);
    if (s != FC_OK) return s;
    s = check_g2_shape(M, K0, N0, N1, act, &rf_ok, &stream_ok);
    if (s != FC_OK) return s;
    if (M == 0) return fail(FC_E_SHAPE, "M == 0: nothing to time");
    if (reps < 1 || reps > 1000) return fail(FC_E_SHAPE, "reps=%d outside 1..1000", (int)reps);
    hipStream_t st = (hipStream_t)stream;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "chain_gemm2_tune: hipGetDevice");
    hipEvent_t t0 = nullptr, t1 = nullptr;
    e = hipEventCreate(&t0);
    if (e == hipSuccess) e = hipEventCreate(&t1);
    float tv[4] = {-1.0f, -1.0f, -1.0f, -1.0f};
    int vbest = -1;
    const int cand[3] = {fc::VARIANT_RF, fc::VARIANT_STREAM, fc::VARIANT_LDS};
    for (int i = 0; i < 3 && e == hipSuccess; ++i) {
        const int v = cand[i];
        if ((v == fc::VARIANT_RF && !rf_ok) || (v == fc::VARIANT_STREAM && !stream_ok)) continue;
        auto launch = [&]() {
            return fc::run_chain_gemm2(H(A), H(W0), H(b0), act, H(W1), H(b1), Hm(D1), M, K0, N0, N1, v, st);
        };
        e = launch();   // untimed: first-use set-up (LDS limits, code upload)
        if (e == hipSuccess) e = hipEventRecord(t0, st);
        for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch();
        if (e == hipSuccess) e = hipEventRecord(t1, st);
        if (e == hipSuccess) e = hipEventSynchronize(t1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
        if (e != hipSuccess) break;
        tv[v] = 1000.0f * ms / (float)reps;
        if (vbest < 0 || tv[v] < tv[vbest]) vbest = v;
    }
    if (t0) (void)hipEventDestroy(t0);
    if (t1) (void)hipEventDestroy(t1);
    if (e != hipSuccess) return hip_status(e, "chain_gemm2_tune");
    tv[FC_VARIANT_AUTO] = tv[vbest];
    {
        std::lock_guard<std::mutex> g(g_tune_mu);
        g_tune[TuneKey(dev, M, K0, N0, N1, (int)act)] = vbest;
    }
    if (best) *best = (fc_variant)vbest;
    if (us)
        for (int i = 0; i < 4; ++i) us[i] = tv[i];
    return ok();
}

fc_status chain_gemm2_auto_variant(int64_t M, int32_t K0, int32_t N0, int32_t N1, fc_act act, fc_variant* out)
{
    bool rf_ok = false, stream_ok = false;
    if (!out) return fail(FC_E_NULL, "out is required");
    fc_status s = check_g2_shape(M, K0, N0, N1, act, &rf_ok, &stream_ok);
    if (s != FC_OK) return s;
    *out = (fc_variant)auto_variant(M, K0, N0, N1, (int)act, rf_ok, stream_ok);
    return ok();
}

void fc_tune_clear(void)
{
    std::lock_guard<std::mutex> g(g_tune_mu);
    g_tune.clear();
}

fc_status chain_gemm2(const fc_half* A, const fc_half* W0, const fc_half* b0, fc_act act, const fc_half* W1,
                      const fc_half* b1, fc_half* D1, int64_t M, int32_t K0, int32_t N0, int32_t N1, void* stream)
{
    return chain_gemm2_variant(A, W0, b0, act, W1, b1, D1, M, K0, N0, N1, FC_VARIANT_AUTO, stream);
}

fc_status chain_gemmN(const fc_half* A, int32_t nstages, const fc_half* const* W, const fc_half* const* b,
                      const fc_act* act, const int32_t* widths, fc_half* D, int64_t M, void* stream)
{
    if (!W || !act || !widths) return fail(FC_E_NULL, "W, act and widths are required");
    if (nstages < 3 || nstages > 4)
        return fail(FC_E_UNSUPPORTED, "nstages=%d: chain_gemmN runs 3 or 4 GEMMs (chain_gemm2 runs 2)", (int)nstages);
    if (M < 0) return fail(FC_E_SHAPE, "M>=0 required");
    for (int i = 0; i <= nstages; ++i) {
        if (widths[i] <= 0 || widths[i] % 8)
            return fail(FC_E_SHAPE, "widths[%d]=%d must be a positive multiple of 8", i, (int)widths[i]);
    }
    if (M > 0 && (!A || !D)) return fail(FC_E_NULL, "A and D are required");
    if (!aligned16(A) || !aligned16(D)) return fail(FC_E_ALIGN, "tensor pointers must be 16-byte aligned");
    const fc_half* Ws[4];
    const fc_half* bs[4];
    int acts[4];
    for (int i = 0; i < nstages; ++i) {
        if (!W[i]) return fail(FC_E_NULL, "W[%d] is required", i);
        const fc_half* bi = b ? b[i] : nullptr;
        if (!aligned16(W[i]) || !aligned16(bi)) return fail(FC_E_ALIGN, "W[%d] and b[%d] must be 16-byte aligned", i, i);
        fc_status s = check_act(act[i]);
        if (s != FC_OK) return s;
        Ws[i] = W[i];
        bs[i] = bi;
        acts[i] = (int)act[i];
    }
    int w[5];
    for (int i = 0; i <= nstages; ++i) w[i] = widths[i];
    if (!fc::gemmn_fits(nstages, w))
        return fail(FC_E_UNSUPPORTED, "register residence: every intermediate width <= 128 and all weights within LDS");
    const fc::half_t* Wh[4];
    const fc::half_t* bh[4];
    for (int i = 0; i < nstages; ++i) {
        Wh[i] = H(Ws[i]);
        bh[i] = H(bs[i]);
    }
    return hip_status(fc::run_chain_gemmN(H(A), nstages, Wh, bh, acts, w, Hm(D), M, (hipStream_t)stream),
                      "chain_gemmN");
}

fc_status gemm_bias_act(const fc_half* A, const fc_half* W, const fc_half* b, fc_act act, fc_half* C, int64_t M,
                        int32_t K, int32_t N, void* stream)
{
    if (M < 0 || K <= 0 || N <= 0) return fail(FC_E_SHAPE, "M>=0 and K, N > 0 required");
    if (!W || (M > 0 && (!A || !C))) return fail(FC_E_NULL, "A, W and C are required");
    if (K % 8 || N % 8) return fail(FC_E_SHAPE, "K and N must be multiples of 8");
    if (!aligned16(A) || !aligned16(W) || !aligned16(C) || !aligned16(b))
        return fail(FC_E_ALIGN, "tensor pointers must be 16-byte aligned");
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    return hip_status(fc::run_gemm_bias_act(H(A), H(W), H(b), act, Hm(C), M, K, N, (hipStream_t)stream),
                      "gemm_bias_act");
}

// conv3x3 -> (x scale) + b -> act -> optional 2x2 pool (scale may be NULL),
// in the kernel form `variant` (fc_conv_variant).
static fc_status conv_pool_impl(const char* name, const fc_half* x, const fc_half* w, const fc_half* scale,
                                const fc_half* b, fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape,
                                uint8_t* argmax, int variant, void* stream)
{
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    if ((int)pool < 0 || (int)pool > 2) return fail(FC_E_ARG, "pool %d out of range", (int)pool);
    if (pool != FC_POOL_MAX_2X2_S2 && argmax) return fail(FC_E_ARG, "argmax needs the max pool");
    if (variant < 0 || variant > 2) return fail(FC_E_ARG, "conv variant %d out of range", variant);
    s = check_conv(shape, 128);
    if (s != FC_OK) return s;
    const long npix = (long)shape->n * shape->h * shape->w;
    const long nout = pool == FC_POOL_NONE ? npix : (long)shape->n * (shape->h / 2) * (shape->w / 2);
    if (!w || (npix > 0 && !x) || (nout > 0 && !y)) return fail(FC_E_NULL, "x, w and y are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned16(b) || !aligned16(scale))
        return fail(FC_E_ALIGN, "tensor pointers must be 16-byte aligned");
    const bool lds_ok = fc::convw_fits(shape->c, shape->k);
    const bool reg_ok = pool != FC_POOL_NONE && fc::conv_pool_wr_fits(shape->w, shape->c, shape->k);
    if (variant == FC_CONV_REG_WEIGHTS && !reg_ok)
        return fail(FC_E_UNSUPPORTED, "register-weights conv needs c == 64, 64 < k <= 128, w*c < 2^27 and a pool");
    if (variant == FC_CONV_LDS_WEIGHTS && !lds_ok) return fail(FC_E_UNSUPPORTED, "weights exceed LDS");
    if (variant == FC_CONV_AUTO && !lds_ok && !reg_ok) return fail(FC_E_UNSUPPORTED, "weights exceed LDS");
    if (nout == 0) return ok();
    const bool regw = variant == FC_CONV_REG_WEIGHTS || (variant == FC_CONV_AUTO && reg_ok);
    hipStream_t st = (hipStream_t)stream;
    if (pool == FC_POOL_NONE)
        return hip_status(fc::run_conv_bias_act3x3(H(x), H(w), H(scale), H(b), act, Hm(y), shape->n, shape->h,
                                                    shape->w, shape->c, shape->k, st),
                          name);
    return hip_status(fc::run_conv_pool3x3(H(x), H(w), H(scale), H(b), act, pool == FC_POOL_AVG_2X2_S2, Hm(y),
                                           argmax, shape->n, shape->h, shape->w, shape->c, shape->k, regw, st),
                      name);
}

fc_status chain_conv_pool(const fc_half* x, const fc_half* w, const fc_half* b, fc_act act, fc_pool pool,
                          fc_half* y, const fc_conv_shape* shape, uint8_t* argmax, void* stream)
{
    return conv_pool_impl(pool == FC_POOL_NONE ? "conv_bias_act" : "chain_conv_pool", x, w, nullptr, b, act, pool, y,
                          shape, argmax, FC_CONV_AUTO, stream);
}

fc_status chain_conv_bn_pool(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* shift,
                             fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape, uint8_t* argmax,
                             void* stream)
{
    if (!scale) return fail(FC_E_NULL, "scale is required (use chain_conv_pool for a plain bias)");
    return conv_pool_impl("chain_conv_bn_pool", x, w, scale, shift, act, pool, y, shape, argmax, FC_CONV_AUTO,
                          stream);
}

fc_status chain_conv_pool_ex(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* shift,
                             fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape, uint8_t* argmax,
                             fc_conv_variant variant, void* stream)
{
    return conv_pool_impl("chain_conv_pool_ex", x, w, scale, shift, act, pool, y, shape, argmax, (int)variant,
                          stream);
}

fc_status conv_bias_act(const fc_half* x, const fc_half* w, const fc_half* b, fc_act act, fc_half* y,
                        const fc_conv_shape* shape, void* stream)
{
    return chain_conv_pool(x, w, b, act, FC_POOL_NONE, y, shape, nullptr, stream);
}

fc_status chain_conv2(const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act, const fc_half* w1,
                      const fc_half* b1, int32_t k1, fc_half* y, const fc_conv_shape* shape0, void* stream)
{
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    if (k1 <= 0 || k1 % 8) return fail(FC_E_SHAPE, "k1=%d must be a positive multiple of 8", k1);
    s = check_conv(shape0, 128);
    if (s != FC_OK) return s;
    const long npix = (long)shape0->n * shape0->h * shape0->w;
    if (!w0 || !w1 || (npix > 0 && (!x || !y))) return fail(FC_E_NULL, "x, w0, w1 and y are required");
    if (!aligned16(x) || !aligned16(w0) || !aligned16(w1) || !aligned16(y) || !aligned16(b0) || !aligned16(b1))
        return fail(FC_E_ALIGN, "tensor pointers must be 16-byte aligned");
    if (npix == 0) return ok();
    if (!fc::rf_fits(9 * shape0->c, shape0->k, k1))
        return fail(FC_E_UNSUPPORTED, "w0 and w1 do not fit in LDS together");
    return hip_status(fc::run_chain_conv2_3x3(H(x), H(w0), H(b0), act, H(w1), H(b1), Hm(y), shape0->n, shape0->h,
                                              shape0->w, shape0->c, shape0->k, k1, (hipStream_t)stream),
                      "chain_conv2");
}

fc_status chain_convN(const fc_half* x, const fc_conv_shape* shape0, int32_t nstages, const fc_half* const* w,
                      const fc_half* const* b, const fc_act* act, const int32_t* k, fc_half* y, void* stream)
{
    if (!w || !act || !k) return fail(FC_E_NULL, "w, act and k are required");
    if (nstages < 3 || nstages > 4)
        return fail(FC_E_UNSUPPORTED, "nstages=%d: chain_convN runs 3 or 4 stages (chain_conv2 runs 2)", (int)nstages);
    fc_status s = check_conv(shape0, 128);
    if (s != FC_OK) return s;
    if (k[0] != shape0->k) return fail(FC_E_SHAPE, "k[0]=%d must equal shape0->k=%d", (int)k[0], (int)shape0->k);
    for (int i = 1; i < nstages; ++i)
        if (k[i] <= 0 || k[i] % 8) return fail(FC_E_SHAPE, "k[%d]=%d must be a positive multiple of 8", i, (int)k[i]);
    const long npix = (long)shape0->n * shape0->h * shape0->w;
    if (npix > 0 && (!x || !y)) return fail(FC_E_NULL, "x and y are required");
    if (!aligned16(x) || !aligned16(y)) return fail(FC_E_ALIGN, "tensor pointers must be 16-byte aligned");
    const fc::half_t* wh[4];
    const fc::half_t* bh[4];
    int acts[4];
    for (int i = 0; i < nstages; ++i) {
        if (!w[i]) return fail(FC_E_NULL, "w[%d] is required", i);
        const fc_half* bi = b ? b[i] : nullptr;
        if (!aligned16(w[i]) || !aligned16(bi)) return fail(FC_E_ALIGN, "w[%d] and b[%d] must be 16-byte aligned", i, i);
        s = check_act(act[i]);
        if (s != FC_OK) return s;
        wh[i] = H(w[i]);
        bh[i] = H(bi);
        acts[i] = (int)act[i];
    }
    int widths[5];
    widths[0] = 9 * shape0->c;
    for (int i = 0; i < nstages; ++i) widths[i + 1] = k[i];
    if (!fc::gemmn_fits(nstages, widths))
        return fail(FC_E_UNSUPPORTED, "register residence: every intermediate width <= 128 and all weights within LDS");
    if (npix == 0) return ok();
    return hip_status(fc::run_chain_convN_3x3(H(x), nstages, wh, bh, acts, widths, Hm(y), shape0->n, shape0->h,
                                              shape0->w, shape0->c, (hipStream_t)stream),
                      "chain_convN");
}

fc_status maxpool2x2(const fc_half* x, fc_half* y, uint8_t* argmax, int32_t n, int32_t h, int32_t w, int32_t c,
                     void* stream)
{
    if (n < 0 || h < 0 || w < 0 || c <= 0 || c % 8) return fail(FC_E_SHAPE, "bad pool shape");
    const long nout = (long)n * (h / 2) * (w / 2);
    if (nout > 0 && (!x || !y)) return fail(FC_E_NULL, "x and y are required");
    if (nout == 0) return ok();
    if (!aligned16(x) || !aligned16(y) || ((uintptr_t)argmax & 7u))
        return fail(FC_E_ALIGN, "x, y 16-byte and argmax 8-byte aligned");
    return hip_status(fc::run_pool2x2(false, H(x), Hm(y), argmax, n, h, w, c, (hipStream_t)stream), "maxpool2x2");
}

fc_status avgpool2x2(const fc_half* x, fc_half* y, int32_t n, int32_t h, int32_t w, int32_t c, void* stream)
{
    if (n < 0 || h < 0 || w < 0 || c <= 0 || c % 8) return fail(FC_E_SHAPE, "bad pool shape");
    const long nout = (long)n * (h / 2) * (w / 2);
    if (nout > 0 && (!x || !y)) return fail(FC_E_NULL, "x and y are required");
    if (nout == 0) return ok();
    if (!aligned16(x) || !aligned16(y)) return fail(FC_E_ALIGN, "x and y must be 16-byte aligned");
    return hip_status(fc::run_pool2x2(true, H(x), Hm(y), nullptr, n, h, w, c, (hipStream_t)stream), "avgpool2x2");
}

fc_status pad_channels(const fc_half* src, fc_half* dst, int64_t outer, int32_t c_in, int32_t c_out, int32_t inner,
                       void* stream)
{
    if (!src || !dst) return fail(FC_E_NULL, "src and dst are required");
    if (outer < 0 || c_in < 0 || c_out < c_in || inner <= 0) return fail(FC_E_SHAPE, "bad padding shape");
    return hip_status(fc::run_pad_mid(H(src), Hm(dst), outer, c_in, c_out, inner, (hipStream_t)stream),
                      "pad_channels");
}

}  // extern "C"
