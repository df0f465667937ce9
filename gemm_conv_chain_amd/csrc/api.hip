// api.hip -- the C ABI of libfusedchain (declared in include/fusedchain.h):
// host-side argument validation, variant choice and launch on the caller's
// stream.  Validation happens before any HIP call.
#include <stdarg.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <vector>

#include "../../include/fusedchain.h"
#include "fc_launch.h"

namespace fc {
hipError_t run_conv_bias_act3x3(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act,
                                half_t* y, int NB, int H, int W, int C, int K, hipStream_t st);
hipError_t run_conv_pool3x3(const half_t* x, const half_t* w, const half_t* scale, const half_t* b, int act,
                            bool avg, half_t* y, uint8_t* argmax, int NB, int H, int W, int C, int K, bool regw,
                            int waves, hipStream_t st);
bool conv_pool_wr_fits(int W, int C, int K);
hipError_t run_chain_conv2_3x3(const half_t* x, const half_t* w0, const half_t* b0, int act, const half_t* w1,
                               const half_t* b1, half_t* y, int NB, int H, int W, int C, int K0, int K1, int waves,
                               int stages, hipStream_t st);
bool conv2_pipe_fits(int W, int C, int K0, int K1);
hipError_t run_chain_conv3_pipe(const half_t* x, const half_t* const* w, const half_t* const* b, const int* act,
                                half_t* y, int NB, int H, int W, int K2, hipStream_t st);
hipError_t run_chain_conv2_pipe(const half_t* x, const half_t* w0, const half_t* b0, int act, const half_t* w1,
                                const half_t* b1, half_t* y, int NB, int H, int W, int K1, hipStream_t st);
hipError_t run_chain_convN_3x3(const half_t* x, int nst, const half_t* const* w, const half_t* const* b,
                               const int* act, const int* widths, half_t* y, int NB, int H, int W, int C,
                               hipStream_t st);
bool gemmn_fits(int nst, const int* widths);
hipError_t run_pool2x2(bool avg, const half_t* v, half_t* y, uint8_t* am, int NB, int P, int Q, int K,
                       hipStream_t st);
hipError_t run_pad_mid(const half_t* src, half_t* dst, long outer, int c_in, int c_out, int inner, hipStream_t st);
bool convw_fits(int C, int K);
bool wino_fits(int C, int K);
hipError_t run_wino_weights(const half_t* w, half_t* U, int C, int K, hipStream_t st);
hipError_t run_conv_pool_wino(const half_t* x, const half_t* U, const half_t* b, int act, bool avg, half_t* y,
                              uint8_t* argmax, int NB, int H, int W, int C, int K, hipStream_t st);
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

// Shapes the conv kernels implement: 3x3, stride 1, pad 1, c % 8, k % 8.
fc_status check_conv(const fc_conv_shape* s, int kmax)
{
    if (!s) return fail(FC_E_NULL, "shape is NULL");
    if (s->n < 0 || s->h < 0 || s->w < 0 || s->c <= 0 || s->k <= 0 || s->r <= 0 || s->s <= 0 || s->stride <= 0 ||
        s->pad < 0)
        return fail(FC_E_SHAPE, "bad conv shape");
    if (s->c % 8 || s->k % 8) return fail(FC_E_SHAPE, "c=%d and k=%d must be multiples of 8", s->c, s->k);
    if (s->r != 3 || s->s != 3 || s->stride != 1 || s->pad != 1)
        return fail(FC_E_UNSUPPORTED, "only 3x3 stride-1 pad-1 convolutions are implemented");
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

// ---- profiled configurations (chain_gemm2_tune_ex, chain_conv_pool_tune):
// kernel form and tile-owning waves per block, cached per device and shape.
struct Config {
    int variant;
    int waves;    // 0: the kernel's own block shape
    int stages;   // register-resident chains: row-chunk ring depth (0: the default 4; 2)
};

// The register-resident kernels come with a two-stage row ring for 4 or 9
// chunks of 64 (k = 193..256 or 513..576).
bool two_stage_ok(int K0)
{
    const int c = (K0 + 63) / 64;
    return c == 4 || c == 9;
}
typedef std::vector<int64_t> TuneKey;   // kind, device, shape ...
std::mutex g_tune_mu;
std::map<TuneKey, Config> g_tune;
enum { TK_GEMM2 = 0, TK_CONV_POOL = 1, TK_CONV2 = 2, TK_CONVN = 3 };

// The cached configuration for key (device appended here), if any.  The
// device is only queried when something has been tuned.
bool tuned_config(TuneKey key, Config* out)
{
    std::lock_guard<std::mutex> g(g_tune_mu);
    if (g_tune.empty()) return false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    key.insert(key.begin() + 1, dev);
    auto it = g_tune.find(key);
    if (it == g_tune.end()) return false;
    *out = it->second;
    return true;
}

void store_config(TuneKey key, int dev, Config c)
{
    key.insert(key.begin() + 1, dev);
    std::lock_guard<std::mutex> g(g_tune_mu);
    g_tune[key] = c;
}

TuneKey gemm2_key(int64_t M, int32_t K0, int32_t N0, int32_t N1, int act) { return {TK_GEMM2, M, K0, N0, N1, act}; }

TuneKey conv_key(const fc_conv_shape* s, int act, int pool, bool argmax)
{
    return {TK_CONV_POOL, s->n, s->h, s->w, s->c, s->k, act, pool, argmax ? 1 : 0};
}

// Candidates of the two-GEMM chain: the register-resident form with 8, 4, 2
// or 1 tile-owning waves per block (a block covers 32 * waves rows per
// round), each with the default four-stage row ring and, where the kernels
// exist (two_stage_ok), a two-stage one; then the streamed-weight and the
// LDS-resident forms (fixed block shapes).  The first applicable one is the
// untuned rule.  At most 10.
int gemm2_candidates(bool rf_ok, bool stream_ok, int K0, Config* out)
{
    int n = 0;
    if (rf_ok) {
        for (int w : {8, 4, 2, 1}) out[n++] = Config{fc::VARIANT_RF, w, 0};
        if (two_stage_ok(K0))
            for (int w : {8, 4, 2, 1}) out[n++] = Config{fc::VARIANT_RF, w, 2};
    }
    if (stream_ok) out[n++] = Config{fc::VARIANT_STREAM, 0, 0};
    out[n++] = Config{fc::VARIANT_LDS, 0, 0};
    return n;
}

// Untuned: the first candidate; for the register-resident form, blocks of
// the smallest power-of-two number of tile-owning waves that covers the
// 32-row tiles with one block per CU (small problems then spread over many
// CUs in small blocks instead of filling a few blocks), and with 8 waves the
// two-stage row ring where it is built (measured: 4-9% faster than four
// stages at 8 waves; fewer waves per block need the deeper ring).
Config gemm2_config(int64_t M, int32_t K0, int32_t N0, int32_t N1, int act, bool rf_ok, bool stream_ok)
{
    Config c;
    if (tuned_config(gemm2_key(M, K0, N0, N1, act), &c)) return c;
    Config cand[16];
    gemm2_candidates(rf_ok, stream_ok, K0, cand);
    c = cand[0];
    if (c.variant == fc::VARIANT_RF) {
        const int64_t tiles = (M + 31) / 32, cus = fc::device_cu_count();
        c.waves = 1;
        while (c.waves < 8 && (int64_t)c.waves * cus < tiles) c.waves *= 2;
        c.stages = c.waves == 8 && two_stage_ok(K0) ? 2 : 0;
    }
    return c;
}

TuneKey conv2_key(const fc_conv_shape* s, int k1, int act)
{
    return {TK_CONV2, s->n, s->h, s->w, s->c, s->k, k1, act};
}

bool conv2_pipe_ok(const fc_conv_shape* s, int k1) { return fc::conv2_pipe_fits(s->w, s->c, s->k, k1); }

TuneKey convN_key(const fc_conv_shape* s, int nst, const int32_t* k)
{
    TuneKey key{TK_CONVN, s->n, s->h, s->w, s->c, nst};
    for (int i = 0; i < 4; ++i) key.push_back(i < nst ? k[i] : 0);
    return key;
}

// Candidates of the conv3x3 -> conv1x1 chain: the pipelined two-group form
// (where it takes the shape), then the register-resident form with 8, 4, 2 or
// 1 tile-owning waves per block, each with the four-stage and (where it
// exists) the two-stage row ring.
int conv2_candidates(const fc_conv_shape* s, int k1, Config* out)
{
    int n = 0;
    if (conv2_pipe_ok(s, k1)) out[n++] = Config{fc::VARIANT_PIPE, 0, 0};
    for (int w : {8, 4, 2, 1}) out[n++] = Config{fc::VARIANT_RF, w, 0};
    if (two_stage_ok(9 * s->c))
        for (int w : {8, 4, 2, 1}) out[n++] = Config{fc::VARIANT_RF, w, 2};
    return n;
}

// Untuned: the pipelined two-group form where it takes the shape (measured
// faster at the 32 x 56 x 56 x 64 -> 64 -> 256 workload); else, as for the
// two-GEMM chain, the smallest power-of-two number of tile-owning waves whose
// blocks, one per CU, cover the 32-pixel tiles (with 8 waves, the two-stage
// row ring where it is built).
Config conv2_config(const fc_conv_shape* s, int k1, int act)
{
    Config c;
    if (tuned_config(conv2_key(s, k1, act), &c)) return c;
    if (conv2_pipe_ok(s, k1)) return Config{fc::VARIANT_PIPE, 0, 0};
    const int64_t tiles = ((int64_t)s->n * s->h * s->w + 31) / 32, cus = fc::device_cu_count();
    c = Config{fc::VARIANT_RF, 1, 0};
    while (c.waves < 8 && (int64_t)c.waves * cus < tiles) c.waves *= 2;
    c.stages = c.waves == 8 && two_stage_ok(9 * s->c) ? 2 : 0;
    return c;
}

// Candidates of the conv + pool chain: the register-weights form (when it
// takes the shape), then the LDS-weights form with 8 or 4 tile-owning waves
// per block (two or one per SIMD).
int conv_candidates(bool lds_ok, bool reg_ok, Config* out)
{
    int n = 0;
    if (reg_ok) out[n++] = Config{FC_CONV_REG_WEIGHTS, 0};
    if (lds_ok)
        for (int w : {8, 4}) out[n++] = Config{FC_CONV_LDS_WEIGHTS, w, 0};
    return n;
}

Config conv_config(const fc_conv_shape* s, int act, int pool, bool argmax, bool lds_ok, bool reg_ok)
{
    Config c;
    if (tuned_config(conv_key(s, act, pool, argmax), &c)) return c;
    Config cand[8];
    conv_candidates(lds_ok, reg_ok, cand);
    return cand[0];
}

// Times `reps` launches of f (after one untimed launch) between two events
// on st; *us = mean microseconds per launch.
template <class F>
hipError_t time_launches(F&& f, int reps, hipStream_t st, hipEvent_t t0, hipEvent_t t1, float* us)
{
    hipError_t e = f();   // untimed: first-use set-up (LDS limits, code upload)
    if (e == hipSuccess) e = hipEventRecord(t0, st);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = f();
    if (e == hipSuccess) e = hipEventRecord(t1, st);
    if (e == hipSuccess) e = hipEventSynchronize(t1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
    if (e == hipSuccess) *us = 1000.0f * ms / (float)reps;
    return e;
}

// Times every candidate config[0 .. n), fills table (up to capacity rows)
// and *best, and caches the fastest under key.
template <class F>
fc_status profile(const char* name, F&& launch, const Config* cand, int n, int reps, const TuneKey& key,
                  fc_tune_entry* table, int32_t capacity, int32_t* count, fc_tune_entry* best, hipStream_t st)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, name);
    hipEvent_t t0 = nullptr, t1 = nullptr;
    e = hipEventCreate(&t0);
    if (e == hipSuccess) e = hipEventCreate(&t1);
    int ib = -1;
    float tb = 0.0f;
    for (int i = 0; i < n && e == hipSuccess; ++i) {
        float us = -1.0f;
        e = time_launches([&]() { return launch(cand[i]); }, reps, st, t0, t1, &us);
        if (e != hipSuccess) break;
        if (table && i < capacity) table[i] = fc_tune_entry{cand[i].variant, cand[i].waves, cand[i].stages, us};
        if (ib < 0 || us < tb) {
            ib = i;
            tb = us;
        }
    }
    if (t0) (void)hipEventDestroy(t0);
    if (t1) (void)hipEventDestroy(t1);
    if (e != hipSuccess) return hip_status(e, name);
    store_config(key, dev, cand[ib]);
    if (count) *count = n;
    if (best) *best = fc_tune_entry{cand[ib].variant, cand[ib].waves, cand[ib].stages, tb};
    // the last launch is not the winner's: run the winner once more, so the
    // output holds what the cached configuration computes
    return hip_status(launch(cand[ib]), name);
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
    Config c{(int)variant, 0, 0};
    if (c.variant == FC_VARIANT_RF && !rf_ok)
        return fail(FC_E_UNSUPPORTED, "register-resident variant needs N0<=128 and W0,W1 within LDS");
    if (c.variant == FC_VARIANT_STREAM && !stream_ok)
        return fail(FC_E_UNSUPPORTED, "streamed variant needs N1<=16128 (biases beside the weight buffers)");
    if (M == 0) return ok();
    if (c.variant == FC_VARIANT_AUTO) c = gemm2_config(M, K0, N0, N1, (int)act, rf_ok, stream_ok);
    return hip_status(fc::run_chain_gemm2(H(A), H(W0), H(b0), act, H(W1), H(b1), Hm(D1), M, K0, N0, N1, c.variant,
                                          c.waves, c.stages, (hipStream_t)stream),
                      "chain_gemm2");
}

fc_status chain_gemm2_ex(const fc_half* A, const fc_half* W0, const fc_half* b0, fc_act act, const fc_half* W1,
                         const fc_half* b1, fc_half* D1, int64_t M, int32_t K0, int32_t N0, int32_t N1,
                         fc_variant variant, int32_t waves, int32_t stages, void* stream)
{
    bool rf_ok = false, stream_ok = false;
    if (M < 0 || K0 <= 0 || N0 <= 0 || N1 <= 0) return fail(FC_E_SHAPE, "M>=0 and K0, N0, N1 > 0 required");
    fc_status s = check_g2_ptrs(A, W0, b0, W1, b1, D1, M);
    if (s != FC_OK) return s;
    s = check_g2_shape(M, K0, N0, N1, act, &rf_ok, &stream_ok);
    if (s != FC_OK) return s;
    if ((int)variant < 1 || (int)variant > 3) return fail(FC_E_ARG, "variant %d: RF, LDS or STREAM", (int)variant);
    if (variant == FC_VARIANT_RF ? (waves < 0 || waves > 8) : waves != 0)
        return fail(FC_E_ARG, "waves=%d: 0..8 for the register-resident form, 0 otherwise", (int)waves);
    if (variant == FC_VARIANT_RF ? (stages != 0 && stages != 2 && stages != 4) : stages != 0)
        return fail(FC_E_ARG, "stages=%d: 0 (= 4), 4 or 2 for the register-resident form, 0 otherwise", (int)stages);
    if (stages == 2 && !two_stage_ok(K0))
        return fail(FC_E_UNSUPPORTED, "the two-stage row ring is built for K0 in 193..256 or 513..576");
    if (variant == FC_VARIANT_RF && !rf_ok)
        return fail(FC_E_UNSUPPORTED, "register-resident variant needs N0<=128 and W0,W1 within LDS");
    if (variant == FC_VARIANT_STREAM && !stream_ok)
        return fail(FC_E_UNSUPPORTED, "streamed variant needs N1<=16128 (biases beside the weight buffers)");
    if (M == 0) return ok();
    return hip_status(fc::run_chain_gemm2(H(A), H(W0), H(b0), act, H(W1), H(b1), Hm(D1), M, K0, N0, N1, (int)variant,
                                          waves, stages == 4 ? 0 : stages, (hipStream_t)stream),
                      "chain_gemm2_ex");
}

fc_status chain_gemm2_tune_ex(const fc_half* A, const fc_half* W0, const fc_half* b0, fc_act act, const fc_half* W1,
                              const fc_half* b1, fc_half* D1, int64_t M, int32_t K0, int32_t N0, int32_t N1,
                              int32_t reps, fc_tune_entry* table, int32_t capacity, int32_t* count,
                              fc_tune_entry* best, void* stream)
{
    bool rf_ok = false, stream_ok = false;
    if (M < 0 || K0 <= 0 || N0 <= 0 || N1 <= 0) return fail(FC_E_SHAPE, "M>=0 and K0, N0, N1 > 0 required");
    fc_status s = check_g2_ptrs(A, W0, b0, W1, b1, D1, M);
    if (s != FC_OK) return s;
    s = check_g2_shape(M, K0, N0, N1, act, &rf_ok, &stream_ok);
    if (s != FC_OK) return s;
    if (M == 0) return fail(FC_E_SHAPE, "M == 0: nothing to time");
    if (reps < 1 || reps > 1000) return fail(FC_E_SHAPE, "reps=%d outside 1..1000", (int)reps);
    if (capacity < 0 || (capacity > 0 && !table)) return fail(FC_E_NULL, "table is required for capacity > 0");
    Config cand[16];
    const int n = gemm2_candidates(rf_ok, stream_ok, K0, cand);
    hipStream_t st = (hipStream_t)stream;
    auto launch = [&](const Config& c) {
        return fc::run_chain_gemm2(H(A), H(W0), H(b0), act, H(W1), H(b1), Hm(D1), M, K0, N0, N1, c.variant, c.waves,
                                   c.stages, st);
    };
    return profile("chain_gemm2_tune", launch, cand, n, reps, gemm2_key(M, K0, N0, N1, (int)act), table, capacity,
                   count, best, st);
}

fc_status chain_gemm2_tune(const fc_half* A, const fc_half* W0, const fc_half* b0, fc_act act, const fc_half* W1,
                           const fc_half* b1, fc_half* D1, int64_t M, int32_t K0, int32_t N0, int32_t N1,
                           int32_t reps, fc_variant* best, float* us, void* stream)
{
    fc_tune_entry table[16], b{};
    int32_t n = 0;
    fc_status s = chain_gemm2_tune_ex(A, W0, b0, act, W1, b1, D1, M, K0, N0, N1, reps, table, 16, &n, &b, stream);
    if (s != FC_OK) return s;
    if (best) *best = (fc_variant)b.variant;
    if (us) {
        for (int i = 0; i < 4; ++i) us[i] = -1.0f;
        for (int i = 0; i < n; ++i) {
            float& u = us[table[i].variant];
            if (u < 0.0f || table[i].us < u) u = table[i].us;
        }
        us[FC_VARIANT_AUTO] = b.us;
    }
    return ok();
}

fc_status chain_gemm2_auto_variant(int64_t M, int32_t K0, int32_t N0, int32_t N1, fc_act act, fc_variant* out)
{
    if (!out) return fail(FC_E_NULL, "out is required");
    fc_tune_entry e;
    fc_status s = chain_gemm2_auto_config(M, K0, N0, N1, act, &e);
    if (s == FC_OK) *out = (fc_variant)e.variant;
    return s;
}

fc_status chain_gemm2_auto_config(int64_t M, int32_t K0, int32_t N0, int32_t N1, fc_act act, fc_tune_entry* out)
{
    bool rf_ok = false, stream_ok = false;
    if (!out) return fail(FC_E_NULL, "out is required");
    fc_status s = check_g2_shape(M, K0, N0, N1, act, &rf_ok, &stream_ok);
    if (s != FC_OK) return s;
    Config c;
    const bool t = tuned_config(gemm2_key(M, K0, N0, N1, (int)act), &c);
    if (!t) c = gemm2_config(M, K0, N0, N1, (int)act, rf_ok, stream_ok);
    *out = fc_tune_entry{c.variant, c.waves, c.stages, -1.0f};
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

// Validation of the conv (+ pool) chain: shapes, pointers, the kernel form.
static fc_status check_conv_pool(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* b,
                                 fc_act act, fc_pool pool, const fc_half* y, const fc_conv_shape* shape,
                                 const uint8_t* argmax, int variant, bool* lds_ok, bool* reg_ok)
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
    *lds_ok = fc::convw_fits(shape->c, shape->k);
    *reg_ok = pool != FC_POOL_NONE && fc::conv_pool_wr_fits(shape->w, shape->c, shape->k);
    if (variant == FC_CONV_REG_WEIGHTS && !*reg_ok)
        return fail(FC_E_UNSUPPORTED, "register-weights conv needs c == 64, 64 < k <= 128, w*c < 2^27 and a pool");
    if (variant == FC_CONV_LDS_WEIGHTS && !*lds_ok) return fail(FC_E_UNSUPPORTED, "weights exceed LDS");
    if (variant == FC_CONV_AUTO && !*lds_ok && !*reg_ok) return fail(FC_E_UNSUPPORTED, "weights exceed LDS");
    return FC_OK;
}

static hipError_t launch_conv_pool(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* b,
                                   fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape, uint8_t* argmax,
                                   Config c, hipStream_t st)
{
    return fc::run_conv_pool3x3(H(x), H(w), H(scale), H(b), act, pool == FC_POOL_AVG_2X2_S2, Hm(y), argmax, shape->n,
                                shape->h, shape->w, shape->c, shape->k, c.variant == FC_CONV_REG_WEIGHTS, c.waves, st);
}

// conv3x3 -> (x scale) + b -> act -> optional 2x2 pool (scale may be NULL),
// in the kernel form `variant` (fc_conv_variant).
static fc_status conv_pool_impl(const char* name, const fc_half* x, const fc_half* w, const fc_half* scale,
                                const fc_half* b, fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape,
                                uint8_t* argmax, int variant, int waves, void* stream)
{
    bool lds_ok = false, reg_ok = false;
    fc_status s = check_conv_pool(x, w, scale, b, act, pool, y, shape, argmax, variant, &lds_ok, &reg_ok);
    if (s != FC_OK) return s;
    if (variant == FC_CONV_LDS_WEIGHTS && pool != FC_POOL_NONE ? (waves < 0 || waves > 8) : waves != 0)
        return fail(FC_E_ARG, "waves=%d: 0..8 for the pooled LDS-weights form, 0 otherwise", (int)waves);
    const long nout = pool == FC_POOL_NONE ? (long)shape->n * shape->h * shape->w
                                           : (long)shape->n * (shape->h / 2) * (shape->w / 2);
    if (nout == 0) return ok();
    hipStream_t st = (hipStream_t)stream;
    if (pool == FC_POOL_NONE)
        return hip_status(fc::run_conv_bias_act3x3(H(x), H(w), H(scale), H(b), act, Hm(y), shape->n, shape->h,
                                                    shape->w, shape->c, shape->k, st),
                          name);
    Config c{variant, waves};
    if (variant == FC_CONV_AUTO) c = conv_config(shape, (int)act, (int)pool, argmax != nullptr, lds_ok, reg_ok);
    return hip_status(launch_conv_pool(x, w, scale, b, act, pool, y, shape, argmax, c, st), name);
}

fc_status chain_conv_pool_tune(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* shift,
                               fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape, uint8_t* argmax,
                               int32_t reps, fc_tune_entry* table, int32_t capacity, int32_t* count,
                               fc_tune_entry* best, void* stream)
{
    bool lds_ok = false, reg_ok = false;
    fc_status s = check_conv_pool(x, w, scale, shift, act, pool, y, shape, argmax, FC_CONV_AUTO, &lds_ok, &reg_ok);
    if (s != FC_OK) return s;
    if (pool == FC_POOL_NONE) return fail(FC_E_ARG, "the profiler times the pooled chains (pool != FC_POOL_NONE)");
    if ((long)shape->n * (shape->h / 2) * (shape->w / 2) == 0) return fail(FC_E_SHAPE, "empty output: nothing to time");
    if (reps < 1 || reps > 1000) return fail(FC_E_SHAPE, "reps=%d outside 1..1000", (int)reps);
    if (capacity < 0 || (capacity > 0 && !table)) return fail(FC_E_NULL, "table is required for capacity > 0");
    Config cand[8];
    const int n = conv_candidates(lds_ok, reg_ok, cand);
    hipStream_t st = (hipStream_t)stream;
    auto launch = [&](const Config& c) { return launch_conv_pool(x, w, scale, shift, act, pool, y, shape, argmax, c, st); };
    return profile("chain_conv_pool_tune", launch, cand, n, reps, conv_key(shape, (int)act, (int)pool, argmax != nullptr),
                   table, capacity, count, best, st);
}

fc_status chain_conv_pool_auto_config(const fc_conv_shape* shape, fc_act act, fc_pool pool, int32_t with_argmax,
                                      fc_tune_entry* out)
{
    if (!out) return fail(FC_E_NULL, "out is required");
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    if ((int)pool < 1 || (int)pool > 2) return fail(FC_E_ARG, "pool %d: a pooled chain is required", (int)pool);
    s = check_conv(shape, 128);
    if (s != FC_OK) return s;
    const bool lds_ok = fc::convw_fits(shape->c, shape->k);
    const bool reg_ok = fc::conv_pool_wr_fits(shape->w, shape->c, shape->k);
    if (!lds_ok && !reg_ok) return fail(FC_E_UNSUPPORTED, "weights exceed LDS");
    const Config c = conv_config(shape, (int)act, (int)pool, with_argmax != 0, lds_ok, reg_ok);
    *out = fc_tune_entry{c.variant, c.waves, c.stages, -1.0f};
    return ok();
}

fc_status chain_conv_pool(const fc_half* x, const fc_half* w, const fc_half* b, fc_act act, fc_pool pool,
                          fc_half* y, const fc_conv_shape* shape, uint8_t* argmax, void* stream)
{
    return conv_pool_impl(pool == FC_POOL_NONE ? "conv_bias_act" : "chain_conv_pool", x, w, nullptr, b, act, pool, y,
                          shape, argmax, FC_CONV_AUTO, 0, stream);
}

fc_status chain_conv_bn_pool(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* shift,
                             fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape, uint8_t* argmax,
                             void* stream)
{
    if (!scale) return fail(FC_E_NULL, "scale is required (use chain_conv_pool for a plain bias)");
    return conv_pool_impl("chain_conv_bn_pool", x, w, scale, shift, act, pool, y, shape, argmax, FC_CONV_AUTO, 0,
                          stream);
}

fc_status chain_conv_pool_ex(const fc_half* x, const fc_half* w, const fc_half* scale, const fc_half* shift,
                             fc_act act, fc_pool pool, fc_half* y, const fc_conv_shape* shape, uint8_t* argmax,
                             fc_conv_variant variant, int32_t waves, void* stream)
{
    return conv_pool_impl("chain_conv_pool_ex", x, w, scale, shift, act, pool, y, shape, argmax, (int)variant, waves,
                          stream);
}

fc_status conv_bias_act(const fc_half* x, const fc_half* w, const fc_half* b, fc_act act, fc_half* y,
                        const fc_conv_shape* shape, void* stream)
{
    return chain_conv_pool(x, w, b, act, FC_POOL_NONE, y, shape, nullptr, stream);
}

static fc_status check_conv2(const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act, const fc_half* w1,
                             const fc_half* b1, int32_t k1, const fc_half* y, const fc_conv_shape* shape0)
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
    if (!fc::rf_fits(9 * shape0->c, shape0->k, k1))
        return fail(FC_E_UNSUPPORTED, "w0 and w1 do not fit in LDS together");
    return FC_OK;
}

static hipError_t run_conv2(const Config& c, const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act,
                            const fc_half* w1, const fc_half* b1, int32_t k1, fc_half* y, const fc_conv_shape* s,
                            hipStream_t st)
{
    if (c.variant == fc::VARIANT_PIPE)
        return fc::run_chain_conv2_pipe(H(x), H(w0), H(b0), act, H(w1), H(b1), Hm(y), s->n, s->h, s->w, k1, st);
    return fc::run_chain_conv2_3x3(H(x), H(w0), H(b0), act, H(w1), H(b1), Hm(y), s->n, s->h, s->w, s->c, s->k, k1,
                                   c.waves, c.stages, st);
}

fc_status chain_conv2_variant(const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act, const fc_half* w1,
                              const fc_half* b1, int32_t k1, fc_half* y, const fc_conv_shape* shape0,
                              fc_variant variant, int32_t waves, int32_t stages, void* stream)
{
    if (variant != FC_VARIANT_AUTO && variant != FC_VARIANT_RF && variant != FC_VARIANT_PIPE)
        return fail(FC_E_ARG, "variant=%d: the conv chain runs FC_VARIANT_AUTO, _RF or _PIPE", (int)variant);
    if (variant == FC_VARIANT_RF ? (waves < 1 || waves > 8) : waves != 0)
        return fail(FC_E_ARG, "waves=%d: 1..8 for FC_VARIANT_RF, else 0", (int)waves);
    if (variant == FC_VARIANT_RF ? (stages != 0 && stages != 2 && stages != 4) : stages != 0)
        return fail(FC_E_ARG, "stages=%d: 4 or 2 (0 = 4) for FC_VARIANT_RF, else 0", (int)stages);
    fc_status s = check_conv2(x, w0, b0, act, w1, b1, k1, y, shape0);
    if (s != FC_OK) return s;
    if (stages == 2 && !two_stage_ok(9 * shape0->c))
        return fail(FC_E_UNSUPPORTED, "the two-stage row ring is built for 9c in 193..256 or 513..576");
    if (variant == FC_VARIANT_PIPE && !conv2_pipe_ok(shape0, k1))
        return fail(FC_E_UNSUPPORTED, "the pipelined form takes c = 64, k0 = 64, k1 <= 256 (c=%d k0=%d k1=%d)",
                    shape0->c, shape0->k, (int)k1);
    if ((long)shape0->n * shape0->h * shape0->w == 0) return ok();
    const Config c = variant == FC_VARIANT_AUTO ? conv2_config(shape0, k1, (int)act)
                                                : Config{(int)variant, waves, stages == 4 ? 0 : stages};
    return hip_status(run_conv2(c, x, w0, b0, act, w1, b1, k1, y, shape0, (hipStream_t)stream), "chain_conv2");
}

fc_status chain_conv2_ex(const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act, const fc_half* w1,
                         const fc_half* b1, int32_t k1, fc_half* y, const fc_conv_shape* shape0, int32_t waves,
                         int32_t stages, void* stream)
{
    if (waves < 0 || waves > 8) return fail(FC_E_ARG, "waves=%d: 1..8, or 0 for the library's choice", (int)waves);
    if (stages != 0 && stages != 2 && stages != 4)
        return fail(FC_E_ARG, "stages=%d: 4 or 2, or 0 for the library's choice", (int)stages);
    if (waves == 0 && stages != 0) return fail(FC_E_ARG, "stages needs an explicit waves");
    return chain_conv2_variant(x, w0, b0, act, w1, b1, k1, y, shape0, waves > 0 ? FC_VARIANT_RF : FC_VARIANT_AUTO,
                               waves, stages, stream);
}

fc_status chain_conv2(const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act, const fc_half* w1,
                      const fc_half* b1, int32_t k1, fc_half* y, const fc_conv_shape* shape0, void* stream)
{
    return chain_conv2_ex(x, w0, b0, act, w1, b1, k1, y, shape0, 0, 0, stream);
}

fc_status chain_conv2_auto_config(const fc_conv_shape* shape0, int32_t k1, fc_act act, fc_tune_entry* out)
{
    if (!shape0 || !out) return fail(FC_E_NULL, "shape0 and out are required");
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    if (k1 <= 0 || k1 % 8) return fail(FC_E_SHAPE, "k1=%d must be a positive multiple of 8", k1);
    s = check_conv(shape0, 128);
    if (s != FC_OK) return s;
    const Config c = conv2_config(shape0, k1, (int)act);
    *out = fc_tune_entry{c.variant, c.waves, c.stages, -1.0f};
    return ok();
}

fc_status chain_conv2_tune(const fc_half* x, const fc_half* w0, const fc_half* b0, fc_act act, const fc_half* w1,
                           const fc_half* b1, int32_t k1, fc_half* y, const fc_conv_shape* shape0, int32_t reps,
                           fc_tune_entry* table, int32_t capacity, int32_t* count, fc_tune_entry* best, void* stream)
{
    fc_status s = check_conv2(x, w0, b0, act, w1, b1, k1, y, shape0);
    if (s != FC_OK) return s;
    if ((long)shape0->n * shape0->h * shape0->w == 0) return fail(FC_E_SHAPE, "empty output: nothing to time");
    if (reps < 1 || reps > 1000) return fail(FC_E_SHAPE, "reps=%d outside 1..1000", (int)reps);
    if (capacity < 0 || (capacity > 0 && !table)) return fail(FC_E_NULL, "table is required for capacity > 0");
    Config cand[16];
    const int n = conv2_candidates(shape0, k1, cand);
    hipStream_t st = (hipStream_t)stream;
    auto launch = [&](const Config& c) { return run_conv2(c, x, w0, b0, act, w1, b1, k1, y, shape0, st); };
    return profile("chain_conv2_tune", launch, cand, n, reps, conv2_key(shape0, k1, (int)act), table, capacity, count,
                   best, st);
}

// shape rules of chain_convN: widths[0..nstages] filled, *pipe_ok = the
// pipelined form applies
static fc_status check_convN_shape(const fc_conv_shape* shape0, int32_t nstages, const int32_t* k, int* widths,
                                   bool* pipe_ok)
{
    if (nstages < 3 || nstages > 4)
        return fail(FC_E_UNSUPPORTED, "nstages=%d: chain_convN runs 3 or 4 stages (chain_conv2 runs 2)", (int)nstages);
    fc_status s = check_conv(shape0, 128);
    if (s != FC_OK) return s;
    if (k[0] != shape0->k) return fail(FC_E_SHAPE, "k[0]=%d must equal shape0->k=%d", (int)k[0], (int)shape0->k);
    for (int i = 1; i < nstages; ++i)
        if (k[i] <= 0 || k[i] % 8) return fail(FC_E_SHAPE, "k[%d]=%d must be a positive multiple of 8", i, (int)k[i]);
    widths[0] = 9 * shape0->c;
    for (int i = 0; i < nstages; ++i) widths[i + 1] = k[i];
    *pipe_ok = nstages == 3 && k[1] == 64 && fc::conv2_pipe_fits(shape0->w, shape0->c, shape0->k, k[2]);
    return FC_OK;
}

fc_status chain_convN_variant(const fc_half* x, const fc_conv_shape* shape0, int32_t nstages, const fc_half* const* w,
                              const fc_half* const* b, const fc_act* act, const int32_t* k, fc_half* y,
                              fc_variant variant, void* stream)
{
    if (variant != FC_VARIANT_AUTO && variant != FC_VARIANT_RF && variant != FC_VARIANT_PIPE)
        return fail(FC_E_ARG, "variant=%d: the conv chain runs FC_VARIANT_AUTO, _RF or _PIPE", (int)variant);
    if (!w || !act || !k) return fail(FC_E_NULL, "w, act and k are required");
    int widths[5];
    bool pipe_ok = false;
    fc_status s = check_convN_shape(shape0, nstages, k, widths, &pipe_ok);
    if (s != FC_OK) return s;
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
    if (variant == FC_VARIANT_PIPE && !pipe_ok)
        return fail(FC_E_UNSUPPORTED, "the pipelined form takes 3 stages with c = 64, k = 64, 64, <= 256");
    bool use_pipe = variant == FC_VARIANT_PIPE || (variant == FC_VARIANT_AUTO && pipe_ok);
    Config tuned;
    if (variant == FC_VARIANT_AUTO && tuned_config(convN_key(shape0, nstages, k), &tuned))
        use_pipe = tuned.variant == fc::VARIANT_PIPE;   // the profiled form (only applicable ones are cached)
    if (!use_pipe && !fc::gemmn_fits(nstages, widths))
        return fail(FC_E_UNSUPPORTED, "register residence: every intermediate width <= 128 and all weights within LDS");
    if (npix == 0) return ok();
    if (use_pipe)
        return hip_status(fc::run_chain_conv3_pipe(H(x), wh, bh, acts, Hm(y), shape0->n, shape0->h, shape0->w, k[2],
                                                   (hipStream_t)stream),
                          "chain_convN");
    return hip_status(fc::run_chain_convN_3x3(H(x), nstages, wh, bh, acts, widths, Hm(y), shape0->n, shape0->h,
                                              shape0->w, shape0->c, (hipStream_t)stream),
                      "chain_convN");
}

fc_status chain_convN_auto_variant(const fc_conv_shape* shape0, int32_t nstages, const int32_t* k, fc_variant* out)
{
    if (!k || !out) return fail(FC_E_NULL, "k and out are required");
    int widths[5];
    bool pipe_ok = false;
    fc_status s = check_convN_shape(shape0, nstages, k, widths, &pipe_ok);
    if (s != FC_OK) return s;
    Config tuned;
    if (tuned_config(convN_key(shape0, nstages, k), &tuned)) {
        *out = (fc_variant)tuned.variant;
        return ok();
    }
    if (pipe_ok) {
        *out = FC_VARIANT_PIPE;
        return ok();
    }
    if (!fc::gemmn_fits(nstages, widths))
        return fail(FC_E_UNSUPPORTED, "register residence: every intermediate width <= 128 and all weights within LDS");
    *out = FC_VARIANT_RF;
    return ok();
}

fc_status chain_convN(const fc_half* x, const fc_conv_shape* shape0, int32_t nstages, const fc_half* const* w,
                      const fc_half* const* b, const fc_act* act, const int32_t* k, fc_half* y, void* stream)
{
    return chain_convN_variant(x, shape0, nstages, w, b, act, k, y, FC_VARIANT_AUTO, stream);
}

fc_status chain_convN_tune(const fc_half* x, const fc_conv_shape* shape0, int32_t nstages, const fc_half* const* w,
                           const fc_half* const* b, const fc_act* act, const int32_t* k, fc_half* y, int32_t reps,
                           fc_tune_entry* table, int32_t capacity, int32_t* count, fc_tune_entry* best, void* stream)
{
    if (!w || !act || !k) return fail(FC_E_NULL, "w, act and k are required");
    int widths[5];
    bool pipe_ok = false;
    fc_status s = check_convN_shape(shape0, nstages, k, widths, &pipe_ok);
    if (s != FC_OK) return s;
    if ((long)shape0->n * shape0->h * shape0->w == 0) return fail(FC_E_SHAPE, "empty output: nothing to time");
    if (reps < 1 || reps > 1000) return fail(FC_E_SHAPE, "reps=%d outside 1..1000", (int)reps);
    if (capacity < 0 || (capacity > 0 && !table)) return fail(FC_E_NULL, "table is required for capacity > 0");
    Config cand[2];
    int n = 0;
    if (pipe_ok) cand[n++] = Config{fc::VARIANT_PIPE, 0, 0};
    if (fc::gemmn_fits(nstages, widths)) cand[n++] = Config{fc::VARIANT_RF, 0, 0};
    if (n == 0)
        return fail(FC_E_UNSUPPORTED, "register residence: every intermediate width <= 128 and all weights within LDS");
    // one validating call per candidate first: argument errors surface as
    // their own status, before any timing
    for (int i = 0; i < n; ++i) {
        s = chain_convN_variant(x, shape0, nstages, w, b, act, k, y, (fc_variant)cand[i].variant, stream);
        if (s != FC_OK) return s;
    }
    hipStream_t st = (hipStream_t)stream;
    auto launch = [&](const Config& c) -> hipError_t {
        const fc_status r = chain_convN_variant(x, shape0, nstages, w, b, act, k, y, (fc_variant)c.variant, stream);
        return r == FC_OK ? hipSuccess : hipErrorLaunchFailure;
    };
    return profile("chain_convN_tune", launch, cand, n, reps, convN_key(shape0, nstages, k), table, capacity, count,
                   best, st);
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

fc_status winograd_weights(const fc_half* w, fc_half* U, int32_t c, int32_t k, void* stream)
{
    if (c <= 0 || k <= 0 || c % 8 || k % 8) return fail(FC_E_SHAPE, "c=%d and k=%d must be positive multiples of 8", c, k);
    if ((long)c * k * 16 >= (1L << 31)) return fail(FC_E_UNSUPPORTED, "16*c*k exceeds 2^31 - 1 elements");
    if (!w || !U) return fail(FC_E_NULL, "w and U are required");
    if (!aligned16(w) || !aligned16(U)) return fail(FC_E_ALIGN, "w and U must be 16-byte aligned");
    return hip_status(fc::run_wino_weights(H(w), Hm(U), c, k, (hipStream_t)stream), "winograd_weights");
}

fc_status chain_conv_pool_winograd(const fc_half* x, const fc_half* U, const fc_half* b, fc_act act, fc_pool pool,
                                   fc_half* y, const fc_conv_shape* shape, uint8_t* argmax, void* stream)
{
    fc_status s = check_act(act);
    if (s != FC_OK) return s;
    if ((int)pool < 0 || (int)pool > 2) return fail(FC_E_ARG, "pool %d out of range", (int)pool);
    if (pool != FC_POOL_MAX_2X2_S2 && argmax) return fail(FC_E_ARG, "argmax needs the max pool");
    s = check_conv(shape, 128);
    if (s != FC_OK) return s;
    if (pool == FC_POOL_NONE)
        return fail(FC_E_UNSUPPORTED, "the Winograd chain pools each 2x2 output tile (pool must be max or avg)");
    if (!fc::wino_fits(shape->c, shape->k))
        return fail(FC_E_UNSUPPORTED, "Winograd kernel: c must be 32 or 64 and k a multiple of 16 up to 128");
    // input halos are addressed from the image's base with 31-bit byte offsets
    if ((long)shape->h * shape->w * shape->c * 2 >= (1L << 31))
        return fail(FC_E_UNSUPPORTED, "an image of %ld bytes: images must stay below 2^31 bytes",
                    (long)shape->h * shape->w * shape->c * 2);
    const long nout = (long)shape->n * (shape->h / 2) * (shape->w / 2);
    if (!U || (nout > 0 && (!x || !y))) return fail(FC_E_NULL, "x, U and y are required");
    if (!aligned16(x) || !aligned16(U) || !aligned16(y) || !aligned16(b) || !aligned16(argmax))
        return fail(FC_E_ALIGN, "tensor pointers (argmax included) must be 16-byte aligned");
    if (nout == 0) return ok();
    return hip_status(fc::run_conv_pool_wino(H(x), H(U), H(b), (int)act, pool == FC_POOL_AVG_2X2_S2, Hm(y), argmax,
                                             shape->n, shape->h, shape->w, shape->c, shape->k, (hipStream_t)stream),
                      "chain_conv_pool_winograd");
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
