/*
 * fusedchain.h -- C ABI of libfusedchain: fused operator chains that keep the
 * intermediate on-chip, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (the pages this library follows):
 *   - BOLT reading notes ("BOLT: Bridging the Gap between Auto-tuners and
 *     Hardware-native Performance"), section "Persistent kernel (GEMM/Conv)
 *     fusion": several GEMMs/convs fused into one kernel under the
 *     threadblock-residence rule (a block computing a tile of the first GEMM
 *     owns all of that GEMM's N, so the second GEMM reads its input from
 *     on-chip storage); register-file-resident and shared-memory-resident
 *     variants; section "Prerequisite: Epilogue fusion" (element-wise op, type
 *     conversion, broadcast vector, partial reduction); section "Templated code
 *     generation" (NHWC layout; tensors padded to 8 fp16 elements = 128 bits).
 *   - Welder reading notes ("Welder: Scheduling Deep Learning Memory Access via
 *     Tile-graph"), sections "Operator-tile and Tile-graph" and "Tile-graph
 *     Scheduling" (Figure 5): Conv -> ReLU -> MaxPool connected through an
 *     on-chip reuse tile; the conv output is never written to global memory.
 *   - Interview page ("Alibaba AI Infra (2)"), question on GEMM/Conv operator
 *     optimisation: implicit GEMM convolution; 1x1 conv = GEMM.
 *
 * Common conventions
 *   - fc_half is an IEEE-754 binary16 bit pattern.  Every tensor pointer is a
 *     DEVICE pointer owned by the caller; the library allocates nothing and keeps
 *     no per-call state, so calls may be issued from several host threads.
 *   - All matrices are row-major.  Conv tensors are NHWC; conv weights are HWIO
 *     (w[r][s][c][k]), i.e. a row-major [(R*S*C) x K] matrix.
 *   - Every call validates its arguments on the host BEFORE any HIP call and
 *     returns a status; nothing is launched when validation fails.  On success
 *     the work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.  Launch failures
 *     return FC_E_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Tensor pointers must be 16-byte aligned; the lengths of the contiguous
 *     (innermost) dimensions -- K0, N0, N1, K, N, C, channel counts -- must be
 *     multiples of 8 (8 fp16 = 128 bits, the widest vector access).  Row counts
 *     (M, batch, spatial sizes) are arbitrary; tails are masked.
 *   - Bias pointers may be NULL (zero bias).  Data pointers of tensors with no
 *     elements (M == 0, an empty batch, a pooled output of zero size) may be
 *     NULL; such calls launch nothing.  Outputs must not alias inputs and are
 *     fully overwritten.
 *   - Accumulation is fp32; each intermediate is rounded once to fp16 (round to
 *     nearest even) after bias and activation; outputs are fp16.
 */
#ifndef FUSEDCHAIN_H
#define FUSEDCHAIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FC_ABI_VERSION 4

typedef uint16_t fc_half;

typedef enum {
    FC_OK = 0,
    FC_E_NULL = 1,        /* a required pointer is NULL */
    FC_E_SHAPE = 2,       /* a size is negative, zero where it must not be, or not a multiple of 8 */
    FC_E_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    FC_E_UNSUPPORTED = 4, /* valid, but outside what the kernels implement (e.g. residence limit) */
    FC_E_HIP = 5,         /* a HIP runtime call failed while launching */
    FC_E_ARG = 6          /* an enum argument is out of range */
} fc_status;

/* Element-wise epilogue activations.  GELU is its tanh form; Hardswish is
 * x * min(max(x + 3, 0), 6) / 6 (BOLT notes, "Enabling deeper operator
 * fusion": Conv2D + BiasAdd + Hardswish in one kernel). */
typedef enum { FC_ACT_NONE = 0, FC_ACT_RELU = 1, FC_ACT_GELU_TANH = 2, FC_ACT_HARDSWISH = 3 } fc_act;
/* 2x2 stride-2 pooling of the conv output in registers: the maximum (Welder
 * notes, Conv+ReLU+MaxPool), or the average -- another partial reduction in
 * the epilogue (BOLT notes, "Prerequisite: Epilogue fusion"): the mean of the
 * window's four fp16-rounded values, rounded once to fp16. */
typedef enum { FC_POOL_NONE = 0, FC_POOL_MAX_2X2_S2 = 1, FC_POOL_AVG_2X2_S2 = 2 } fc_pool;
typedef enum {
    FC_VARIANT_AUTO = 0,
    FC_VARIANT_RF = 1,
    FC_VARIANT_LDS = 2,
    FC_VARIANT_STREAM = 3,
    FC_VARIANT_PIPE = 4   /* conv3x3 -> conv1x1 (-> conv1x1) only: chain_conv2_variant, chain_convN_variant */
} fc_variant;

/* Kernel forms of the conv + activation + 2x2 pool chain (chain_conv_pool_ex).
 * Both keep the conv output in registers and compute the same values up to
 * fp32 summation order:
 *   FC_CONV_LDS_WEIGHTS  the HWIO weights resident in LDS, rows of pixels
 *                        streamed from global memory into registers (every
 *                        shape chain_conv_pool accepts);
 *   FC_CONV_REG_WEIGHTS  the weights resident in registers as matrix-core
 *                        operands, the input halo of each tile streamed into
 *                        LDS (c == 64, 64 < k <= 128, a max or average pool);
 *   FC_CONV_AUTO         the choice chain_conv_pool_tune cached for the shape,
 *                        else REG_WEIGHTS where it applies, else LDS_WEIGHTS. */
typedef enum { FC_CONV_AUTO = 0, FC_CONV_LDS_WEIGHTS = 1, FC_CONV_REG_WEIGHTS = 2 } fc_conv_variant;

/* x NHWC [n,h,w,c]; w HWIO [r,s,c,k]; output spatial size
 * P = (h + 2*pad - r)/stride + 1, Q = (w + 2*pad - s)/stride + 1. */
typedef struct {
    int32_t n, h, w, c, k, r, s, stride, pad;
} fc_conv_shape;

/* Version of this ABI (FC_ABI_VERSION). */
int32_t fc_abi_version(void);

/* Static, human-readable name of a status code. */
const char *fc_status_str(fc_status s);

/* Detail message of the last failed call on the calling host thread ("" if
 * none).  The pointer stays valid until the thread's next call. */
const char *fc_last_error(void);

/*
 * chain_gemm2 -- D1 = act(A*W0 + b0) * W1 + b1 in one kernel
 * (BOLT notes, "Persistent kernel (GEMM/Conv) fusion").
 *   A  [M  x K0]   W0 [K0 x N0]   b0 [N0]
 *   W1 [N0 x N1]   b1 [N1]        D1 [M  x N1]
 *   act: FC_ACT_NONE / FC_ACT_RELU / FC_ACT_GELU_TANH (tanh form) / FC_ACT_HARDSWISH.
 * The intermediate H = fp16(act(A*W0 + b0)) [M x N0] never reaches global
 * memory.  Residence: one block owns all N0 columns, so N0 <= 256
 * (FC_E_UNSUPPORTED above).  M == 0 is a no-op.
 * Variant (chain_gemm2_variant): FC_VARIANT_RF keeps H in VGPRs with W0, W1
 * resident in LDS (N0 <= 128 and W0, W1 fit in LDS together);
 * FC_VARIANT_LDS stages the GEMM0 accumulator tile through LDS into GEMM1
 * (shared-memory-resident fusion, same notes; N0 <= 256); FC_VARIANT_STREAM
 * keeps H in VGPRs and streams W0, W1 through LDS (N0 <= 256, and N1 <= 16128
 * so the biases fit beside the weight buffers).  FC_VARIANT_AUTO (chain_gemm2)
 * picks RF when it applies, else STREAM, else LDS.  All variants compute the
 * same values up to fp32 summation order.
 */
fc_status chain_gemm2(const fc_half *A, const fc_half *W0, const fc_half *b0, fc_act act,
                      const fc_half *W1, const fc_half *b1, fc_half *D1,
                      int64_t M, int32_t K0, int32_t N0, int32_t N1, void *stream);
fc_status chain_gemm2_variant(const fc_half *A, const fc_half *W0, const fc_half *b0, fc_act act,
                              const fc_half *W1, const fc_half *b1, fc_half *D1,
                              int64_t M, int32_t K0, int32_t N0, int32_t N1,
                              fc_variant variant, void *stream);
/* chain_gemm2_ex -- one explicit configuration, as the profiler times it:
 * variant (not AUTO) and, for FC_VARIANT_RF, waves = tile-owning waves per
 * block, 1..8 (0 = 8), and stages = row-chunk ring depth, 4 (or 0) or 2 (2
 * is built for K0 in 193..256 and 513..576, else FC_E_UNSUPPORTED); other
 * variants take waves == 0 and stages == 0.  FC_E_ARG otherwise. */
fc_status chain_gemm2_ex(const fc_half *A, const fc_half *W0, const fc_half *b0, fc_act act,
                         const fc_half *W1, const fc_half *b1, fc_half *D1,
                         int64_t M, int32_t K0, int32_t N0, int32_t N1,
                         fc_variant variant, int32_t waves, int32_t stages, void *stream);

/*
 * chain_gemm2_tune -- hardware profiling of the fused-chain variants for one
 * shape (BOLT notes, "Light-weight performance profiler": candidate kernel
 * configurations are measured on the GPU and the fastest is kept; Welder
 * notes, "Tile-graph Scheduling": a few efficient tile configurations are
 * profiled on the hardware and the best one chosen).  The candidates are the
 * residence forms of chain_gemm2_variant that apply to (K0, N0, N1).
 * Arguments as for chain_gemm2, plus:
 *   reps     timed launches per candidate, 1..1000 (one untimed launch first);
 *   best     out (host, may be NULL): the fastest variant;
 *   us       out (host, may be NULL): float[4], mean microseconds per launch
 *            indexed by fc_variant (us[FC_VARIANT_AUTO] = the best time;
 *            -1 for a variant that does not apply).
 * The result is cached per (device, M, K0, N0, N1, act): later chain_gemm2 /
 * FC_VARIANT_AUTO calls of that shape run the chosen variant (the cache is
 * process-wide, guarded by a lock).  D1 is overwritten with the chain's
 * result (every candidate computes it).  BLOCKING: the call records HIP
 * events on `stream` and waits for them, so it must not be issued during
 * stream capture.  Validation errors as chain_gemm2; FC_E_SHAPE if reps is
 * out of range; FC_E_SHAPE if M == 0 (nothing to time).
 */
fc_status chain_gemm2_tune(const fc_half *A, const fc_half *W0, const fc_half *b0, fc_act act,
                           const fc_half *W1, const fc_half *b1, fc_half *D1,
                           int64_t M, int32_t K0, int32_t N0, int32_t N1,
                           int32_t reps, fc_variant *best, float *us, void *stream);

/* One timed configuration of the profiler: the kernel form (fc_variant for
 * the GEMM chains, fc_conv_variant for the conv chains), the number of waves
 * per block that own row tiles (0: the form's own block shape; the
 * register-resident GEMM chain takes 8, 4, 2 or 1 -- a block then covers
 * 32 * waves rows per round -- and the LDS-weights conv 8 or 4), the
 * pipeline stages of the register-resident chains' row stream (0: the
 * default ring of 4 chunks, three in flight; 2: two chunks, one in flight;
 * the BOLT profiler's "stages" parameter), and the mean microseconds per
 * launch (-1 where nothing was timed). */
typedef struct {
    int32_t variant;
    int32_t waves;
    int32_t stages;
    float us;
} fc_tune_entry;

/*
 * chain_gemm2_tune_ex -- as chain_gemm2_tune, over every configuration the
 * library can run for the shape (each residence form; the register-resident
 * one with 8, 4, 2 and 1 tile-owning waves per block, each with 4 and, where
 * built, 2 pipeline stages: at most 10 configurations).  table (host, may be
 * NULL when capacity == 0) receives min(count, capacity) rows in the order
 * timed; count (host, may be NULL) the number of configurations timed; best
 * (host, may be NULL) the fastest, which is cached for the shape and runs
 * under FC_VARIANT_AUTO.  D1 holds the chain's result on return.  BLOCKING,
 * like chain_gemm2_tune.  FC_E_NULL if capacity > 0 and table is NULL.
 */
fc_status chain_gemm2_tune_ex(const fc_half *A, const fc_half *W0, const fc_half *b0, fc_act act,
                              const fc_half *W1, const fc_half *b1, fc_half *D1,
                              int64_t M, int32_t K0, int32_t N0, int32_t N1, int32_t reps,
                              fc_tune_entry *table, int32_t capacity, int32_t *count, fc_tune_entry *best,
                              void *stream);

/* The configuration FC_VARIANT_AUTO runs for this shape on the current
 * device (us = -1): the tuned one, else the static rule -- register-resident
 * when it applies, with the smallest power-of-two number of tile-owning waves
 * (1..8) that covers ceil(M / 32) row tiles with one block per CU (with 8
 * waves, 2 pipeline stages where built); else STREAM; else LDS.  Host only. */
fc_status chain_gemm2_auto_config(int64_t M, int32_t K0, int32_t N0, int32_t N1, fc_act act, fc_tune_entry *out);

/* The variant FC_VARIANT_AUTO runs for this shape on the current device:
 * the tuned choice if chain_gemm2_tune cached one, else the static rule (RF
 * when it applies, else STREAM, else LDS).  Host only, launches nothing.
 * Returns FC_E_SHAPE / FC_E_ARG / FC_E_UNSUPPORTED as chain_gemm2 would. */
fc_status chain_gemm2_auto_variant(int64_t M, int32_t K0, int32_t N0, int32_t N1, fc_act act, fc_variant *out);

/* Forget every tuned choice (all devices, GEMM and conv chains). */
void fc_tune_clear(void);

/*
 * chain_gemmN -- an N-stage chain of GEMMs in one kernel, every intermediate
 * kept in registers (BOLT notes, "Persistent kernel (GEMM/Conv) fusion":
 * persistent fusion of more than two GEMMs, MLP-style):
 *   X_0 = A [M x widths[0]];  X_{i+1} = act[i](X_i * W[i] + b[i]),
 *   W[i] [widths[i] x widths[i+1]] row-major, b[i] [widths[i+1]] (b or b[i]
 *   may be NULL), every X_i with 0 < i < nstages rounded once to fp16,
 *   D = X_nstages [M x widths[nstages]] (fp16, rounded once).
 * nstages is 3 or 4 (two GEMMs: chain_gemm2, whose last GEMM has no
 * activation -- pass FC_ACT_NONE as the last act to match it).  Residence:
 * widths[1..nstages-1] <= 128 and all weights within LDS, else
 * FC_E_UNSUPPORTED.  The arrays are host arrays read during the call; W[i],
 * b[i], A and D are device pointers owned by the caller.  M == 0 is a no-op.
 */
fc_status chain_gemmN(const fc_half *A, int32_t nstages, const fc_half *const *W, const fc_half *const *b,
                      const fc_act *act, const int32_t *widths, fc_half *D, int64_t M, void *stream);

/*
 * chain_conv_pool -- y = maxpool2x2(act(conv(x, w) + b)) with the conv output
 * kept in registers (Welder notes, Conv+ReLU+MaxPool tile graph, Figure 5).
 *   x NHWC [n,h,w,c], w HWIO [3,3,c,k], b [k];
 *   pool == FC_POOL_MAX_2X2_S2: y [n, P/2, Q/2, k] (floor), argmax (nullable,
 *   uint8 [n, P/2, Q/2, k]) = 2*dy + dx of the first maximum in the order
 *   (0,0),(0,1),(1,0),(1,1), decided on the fp16-rounded values;
 *   pool == FC_POOL_AVG_2X2_S2: y [n, P/2, Q/2, k] = fp16 of the mean of each
 *   window's four fp16 values (argmax must be NULL);
 *   pool == FC_POOL_NONE: y [n, P, Q, k] = act(conv + b) (argmax must be NULL).
 * Implemented shapes: r = s = 3, stride 1, pad 1, c % 8 == 0 (pad other channel
 * counts with pad_channels first), k % 8 == 0 and k <= 128 (all output channels in
 * one block), n*h*w < 2^31, and the weights, held in LDS for the whole
 * kernel, within 160 KiB: roundup(k,32) * (roundup(9c,64) + 8) * 2 bytes
 * (c = 64: k <= 128; c = 128: k <= 64).  Others: FC_E_UNSUPPORTED.
 */
fc_status chain_conv_pool(const fc_half *x, const fc_half *w, const fc_half *b, fc_act act, fc_pool pool,
                          fc_half *y, const fc_conv_shape *shape, uint8_t *argmax, void *stream);

/*
 * chain_conv_bn_pool -- chain_conv_pool with a per-channel scale before the
 * shift: the inference form of batch normalisation, which the interview
 * page's inference simplification replaces by a scale and a bias
 * (scale = gamma / sqrt(var + eps), shift = beta - mean * scale, computed by
 * the caller), fused into the conv epilogue (BOLT notes, "Prerequisite:
 * Epilogue fusion": broadcast vectors in the epilogue):
 *   v[n,p,q,k] = act(conv3x3(x, w)[n,p,q,k] * scale[k] + shift[k])   (one fp32 fma)
 *   y = maxpool2x2(fp16(v)) (FC_POOL_MAX_2X2_S2), or fp16(v) (FC_POOL_NONE).
 * scale [k] is required (any sign); shift may be NULL.  Everything else --
 * shapes, argmax, alignment, errors -- as chain_conv_pool.
 */
fc_status chain_conv_bn_pool(const fc_half *x, const fc_half *w, const fc_half *scale, const fc_half *shift,
                             fc_act act, fc_pool pool, fc_half *y, const fc_conv_shape *shape,
                             uint8_t *argmax, void *stream);

/*
 * chain_conv_pool_ex -- chain_conv_pool (scale == NULL: shift is the bias) or
 * chain_conv_bn_pool (scale != NULL) with an explicit kernel form
 * (fc_conv_variant) and, for FC_CONV_LDS_WEIGHTS with a pool, the number of
 * tile-owning waves per block (1..8; 0 = 8); other forms take waves == 0.
 * FC_E_UNSUPPORTED if the requested form does not take the shape or the pool
 * (FC_CONV_REG_WEIGHTS needs c == 64, 64 < k <= 128, w * c < 2^27 and
 * pool != FC_POOL_NONE); FC_E_ARG for an unknown form or a bad waves value.
 * Everything else as chain_conv_pool.
 */
fc_status chain_conv_pool_ex(const fc_half *x, const fc_half *w, const fc_half *scale, const fc_half *shift,
                             fc_act act, fc_pool pool, fc_half *y, const fc_conv_shape *shape, uint8_t *argmax,
                             fc_conv_variant variant, int32_t waves, void *stream);

/*
 * chain_conv_pool_tune -- hardware profiling of the pooled conv chain for one
 * shape (BOLT notes, "Light-weight performance profiler"; Welder notes,
 * "Tile-graph Scheduling": candidate configurations measured on the GPU, the
 * fastest kept): times the register-weights form (where it takes the shape)
 * and the LDS-weights form with 8 and 4 tile-owning waves per block, reps
 * launches each after one untimed launch, on the caller's buffers, and
 * caches the fastest for (device, n, h, w, c, k, act, pool, argmax != NULL):
 * chain_conv_pool / chain_conv_bn_pool / FC_CONV_AUTO then run it.
 * Arguments as chain_conv_pool_ex (scale may be NULL), pool must be a 2x2
 * pool, plus reps (1..1000), table / capacity / count / best as
 * chain_gemm2_tune_ex.  y (and argmax) hold the chain's result on return.
 * BLOCKING (waits for its own events; not during stream capture).
 */
fc_status chain_conv_pool_tune(const fc_half *x, const fc_half *w, const fc_half *scale, const fc_half *shift,
                               fc_act act, fc_pool pool, fc_half *y, const fc_conv_shape *shape, uint8_t *argmax,
                               int32_t reps, fc_tune_entry *table, int32_t capacity, int32_t *count,
                               fc_tune_entry *best, void *stream);

/* The configuration FC_CONV_AUTO runs for this pooled shape on the current
 * device (us = -1): the tuned one, else the register-weights form where it
 * applies, else the LDS-weights form with 8 waves.  with_argmax: whether the
 * call passes an argmax output (a different kernel).  Host only. */
fc_status chain_conv_pool_auto_config(const fc_conv_shape *shape, fc_act act, fc_pool pool, int32_t with_argmax,
                                      fc_tune_entry *out);

/*
 * chain_conv2 -- y = conv1x1(act(conv(x, w0) + b0), w1) + b1, the first conv's
 * output kept on chip (BOLT persistent conv fusion; a 1x1 conv is a GEMM,
 * interview page, conv item 5), rounded once to fp16.
 *   x NHWC [n,h,w,c], w0 HWIO [3,3,c,k0] (k0 = shape0->k), b0 [k0],
 *   w1 [k0 x k1] (= HWIO [1,1,k0,k1]), b1 [k1], y NHWC [n,P,Q,k1].
 * Implemented: r = s = 3, stride 1, pad 1, c % 8 == 0, k0 % 8 == 0 and
 * k0 <= 128, k1 % 8 == 0, n*h*w < 2^31, and both weights fit in LDS together.
 * Two kernel forms (chain_conv2_variant): FC_VARIANT_RF keeps the first conv's
 * output in the VGPRs of the wave that computed it (any shape above);
 * FC_VARIANT_PIPE runs the two convs in two pipelined wave groups of one block
 * per CU -- the 3x3 conv's weights in registers, its input halo streamed into
 * LDS by LDS-DMA, the intermediate tile in LDS for the 1x1 conv of the other
 * group -- for c = 64, k0 = 64, k1 <= 256 and w * c < 2^27.  The library
 * runs the profiled form if chain_conv2_tune ran for the shape, else
 * FC_VARIANT_PIPE where it applies, else FC_VARIANT_RF.  Both compute the same
 * values up to the fp32 summation order.
 */
fc_status chain_conv2(const fc_half *x, const fc_half *w0, const fc_half *b0, fc_act act,
                      const fc_half *w1, const fc_half *b1, int32_t k1, fc_half *y,
                      const fc_conv_shape *shape0, void *stream);

/* chain_conv2_ex -- chain_conv2 with the FC_VARIANT_RF block shape chosen by
 * the caller: waves = tile-owning waves per block (1..8; a block's round covers
 * 32 * waves pixels) and stages = row-chunk ring depth (4, or 2 where built:
 * 9c in 193..256 or 513..576, else FC_E_UNSUPPORTED; 0 = 4), or waves =
 * stages = 0 for the library's choice (as chain_conv2; the untuned rule of
 * FC_VARIANT_RF is the smallest power of two whose blocks, one per CU, cover
 * the 32-pixel tiles, with 2 stages at 8 waves where built).  Other values ->
 * FC_E_ARG. */
fc_status chain_conv2_ex(const fc_half *x, const fc_half *w0, const fc_half *b0, fc_act act, const fc_half *w1,
                         const fc_half *b1, int32_t k1, fc_half *y, const fc_conv_shape *shape0, int32_t waves,
                         int32_t stages, void *stream);

/* chain_conv2_variant -- chain_conv2 with the kernel form chosen by the
 * caller: FC_VARIANT_AUTO (waves = stages = 0: the library's choice),
 * FC_VARIANT_RF (waves, stages as chain_conv2_ex, waves >= 1) or
 * FC_VARIANT_PIPE (waves = stages = 0; FC_E_UNSUPPORTED outside its shapes).
 * Other variants or values -> FC_E_ARG; errors otherwise as chain_conv2. */
fc_status chain_conv2_variant(const fc_half *x, const fc_half *w0, const fc_half *b0, fc_act act,
                              const fc_half *w1, const fc_half *b1, int32_t k1, fc_half *y,
                              const fc_conv_shape *shape0, fc_variant variant, int32_t waves, int32_t stages,
                              void *stream);

/* The configuration chain_conv2 runs for this shape on the current device
 * (variant FC_VARIANT_PIPE or FC_VARIANT_RF with waves and stages; us = -1):
 * the tuned one, else the untuned rule of chain_conv2.  Host only. */
fc_status chain_conv2_auto_config(const fc_conv_shape *shape0, int32_t k1, fc_act act, fc_tune_entry *out);

/* chain_conv2_tune -- the profiler of chain_conv2 (BOLT notes, "Light-weight
 * performance profiler"): times reps launches (1..1000, after one untimed
 * launch) of each candidate -- FC_VARIANT_PIPE where it applies, and each
 * FC_VARIANT_RF block shape (8, 4, 2, 1 tile-owning waves) with 4 and, where
 * built, 2 pipeline stages -- on this input, writes up to capacity rows of table
 * (us = mean microseconds per launch), *count = candidates timed, *best = the
 * fastest, and caches it for (device, shape, k1, act): chain_conv2 and
 * chain_conv2_ex(waves = 0) then run it.  y is written (by the winner last).
 * Synchronises the stream.  Errors as chain_conv2; an empty output ->
 * FC_E_SHAPE. */
fc_status chain_conv2_tune(const fc_half *x, const fc_half *w0, const fc_half *b0, fc_act act, const fc_half *w1,
                           const fc_half *b1, int32_t k1, fc_half *y, const fc_conv_shape *shape0, int32_t reps,
                           fc_tune_entry *table, int32_t capacity, int32_t *count, fc_tune_entry *best,
                           void *stream);

/*
 * chain_convN -- a 3x3 convolution followed by 1x1 convolutions in one
 * kernel, every intermediate kept in registers (BOLT notes, "Persistent
 * kernel (GEMM/Conv) fusion": several convolutions fused under the
 * threadblock-residence rule; interview page, Conv item 5: a 1x1 conv is a
 * GEMM over the pixels):
 *   X_1     = act[0](conv3x3(x, w[0]) + b[0])      shape0: x [n,h,w,c], w[0] HWIO [3,3,c,k[0]]
 *   X_{i+1} = act[i](X_i * w[i] + b[i])            1x1: w[i] [k[i-1] x k[i]] (= HWIO [1,1,k[i-1],k[i]])
 *   y       = X_nstages                            [n, h, w, k[nstages-1]]
 * for i = 1 .. nstages-1; each X_i with i < nstages rounded once to fp16.
 * k (host array, nstages entries): output channels of every stage, k[0] ==
 * shape0->k.  nstages is 3 or 4 (two stages: chain_conv2).  shape0 follows
 * chain_conv_pool's rules (3x3, stride 1, pad 1, c % 8 == 0, k[0] <= 128);
 * k[1 .. nstages-2] <= 128 and all weights must fit in LDS together, else
 * FC_E_UNSUPPORTED -- except three stages with c = 64 and k = {64, 64, <= 256},
 * which run the pipelined form (chain_convN_variant, FC_VARIANT_PIPE) and may
 * exceed that LDS rule; after chain_convN_tune for the shape, the profiled form
 * runs instead.  b or b[i] may be NULL.  w, b, act and k are host
 * arrays read during the call; the tensors are device pointers owned by the
 * caller.  An empty batch is a no-op.
 */
fc_status chain_convN(const fc_half *x, const fc_conv_shape *shape0, int32_t nstages,
                      const fc_half *const *w, const fc_half *const *b, const fc_act *act,
                      const int32_t *k, fc_half *y, void *stream);

/* chain_convN_variant -- chain_convN with the kernel form chosen by the caller:
 * FC_VARIANT_AUTO (the pipelined form where it applies, else the register-
 * resident one), FC_VARIANT_RF (the register-resident chain, k_chain_rf with
 * the conv loader: every shape chain_convN takes) or FC_VARIANT_PIPE (three
 * stages only, c = 64, k = {64, 64, <= 256}, w * c < 2^27: the two pipelined
 * wave groups of chain_conv2's FC_VARIANT_PIPE, the middle 1x1 conv run by the
 * 3x3 conv's group one tile behind; FC_E_UNSUPPORTED outside those shapes).
 * Other variants -> FC_E_ARG; errors otherwise as chain_convN. */
fc_status chain_convN_variant(const fc_half *x, const fc_conv_shape *shape0, int32_t nstages,
                              const fc_half *const *w, const fc_half *const *b, const fc_act *act,
                              const int32_t *k, fc_half *y, fc_variant variant, void *stream);

/* The variant chain_convN runs for this shape on the current device: the
 * profiled one if chain_convN_tune ran for the shape, else FC_VARIANT_PIPE
 * where the pipelined form applies, else FC_VARIANT_RF.  Host only, launches
 * nothing; shape errors as chain_convN (FC_E_NULL for a NULL k or out). */
fc_status chain_convN_auto_variant(const fc_conv_shape *shape0, int32_t nstages, const int32_t *k,
                                   fc_variant *out);

/* chain_convN_tune -- time each kernel form chain_convN can run for these
 * tensors (the pipelined form where it applies, the register-resident form
 * where it fits; reps launches each after one untimed launch, on stream,
 * blocking), write one row per form to table (up to capacity rows; *count =
 * forms timed), the fastest to *best, and cache it for the shape (device,
 * n, h, w, c, k[]): chain_convN with FC_VARIANT_AUTO then runs it.  y holds
 * the winner's output on return.  BOLT notes, "Light-weight performance
 * profiler".  Errors as chain_convN; reps outside 1..1000 or an empty batch
 * -> FC_E_SHAPE; capacity > 0 with a NULL table -> FC_E_NULL. */
fc_status chain_convN_tune(const fc_half *x, const fc_conv_shape *shape0, int32_t nstages,
                           const fc_half *const *w, const fc_half *const *b, const fc_act *act,
                           const int32_t *k, fc_half *y, int32_t reps, fc_tune_entry *table, int32_t capacity,
                           int32_t *count, fc_tune_entry *best, void *stream);

/* ---- unfused single-operator kernels (the two-kernel baselines) ---- */

/* C [M x N] = act(A [M x K] * W [K x N] + b [N]), fp16 out (GEMM + epilogue). */
fc_status gemm_bias_act(const fc_half *A, const fc_half *W, const fc_half *b, fc_act act, fc_half *C,
                        int64_t M, int32_t K, int32_t N, void *stream);

/* y NHWC [n,P,Q,k] = act(conv(x, w) + b); same shape limits as chain_conv_pool. */
fc_status conv_bias_act(const fc_half *x, const fc_half *w, const fc_half *b, fc_act act, fc_half *y,
                        const fc_conv_shape *shape, void *stream);

/* y [n, h/2, w/2, c] = 2x2 stride-2 max pool of x NHWC [n,h,w,c] (floor);
 * argmax nullable (8-byte aligned), encoded as in chain_conv_pool. */
fc_status maxpool2x2(const fc_half *x, fc_half *y, uint8_t *argmax, int32_t n, int32_t h, int32_t w, int32_t c,
                     void *stream);

/* y [n, h/2, w/2, c] = 2x2 stride-2 average pool of x NHWC [n,h,w,c] (floor):
 * the mean of each window's four fp16 values, rounded once to fp16 -- the
 * unfused baseline of FC_POOL_AVG_2X2_S2 (BOLT notes, "Prerequisite: Epilogue
 * fusion").  c % 8 == 0; x and y 16-byte aligned. */
fc_status avgpool2x2(const fc_half *x, fc_half *y, int32_t n, int32_t h, int32_t w, int32_t c, void *stream);

/* ---- Winograd F(2x2, 3x3) conv + pool (interview page, "Conv optimisation",
 *      item 3: (m + r - 1)^2 = 16 products per 2x2 output tile of a 3x3
 *      filter instead of m^2 r^2 = 36, paid for with transforms and a small
 *      loss of precision; the transforms are Lavin and Gray's minimal
 *      filtering algorithm: U = G g G^T, V = B^T d B, Y = A^T [sum_c U.V] A) ----
 *
 * winograd_weights -- the transformed weights U = G g G^T of every (c, k),
 * computed exactly (fp64) and rounded once to fp16.
 *   w: HWIO [3, 3, c, k] (device); U: 16*c*k fp16 (device, caller-owned),
 *   written in the library's operand layout [16][c/8][k][8]: U[xi][nu][c][k]
 *   at (((4 xi + nu) * (c/8) + c/8) * k + k) * 8 + c % 8.  Compute once per
 *   weight tensor and pass to chain_conv_pool_winograd.
 *   c, k > 0 and multiples of 8 (else FC_E_SHAPE); 16*c*k < 2^31
 *   (FC_E_UNSUPPORTED); NULL -> FC_E_NULL; pointers 16-byte aligned. */
fc_status winograd_weights(const fc_half *w, fc_half *U, int32_t c, int32_t k, void *stream);

/* chain_conv_pool_winograd -- y = pool2x2(act(conv(x, w) + b)) with the 3x3
 * conv evaluated by F(2x2, 3x3) from U = winograd_weights(w): each 2x2
 * Winograd output tile is one pool window (Welder notes, Conv + ReLU +
 * MaxPool tile graph, Figure 5), so the conv output stays in registers.
 * Numerics: V = B^T d B in fp16 arithmetic (rows first, one rounding per
 * stage), the 16 channel contractions on the matrix cores with fp32
 * accumulation, A^T M A + bias + act in fp32, one rounding to fp16; the pool
 * and argmax as for chain_conv_pool (argmax on the fp16 values, first maximum
 * in the order (0,0),(0,1),(1,0),(1,1)).  The result differs from the direct
 * conv by the rounding of U and V (the precision loss the page names).
 *   x NHWC [n,h,w,c]; U as written by winograd_weights for (c, k); b [k] or
 *   NULL; y [n, h/2, w/2, k] (floor); argmax (max pool only, nullable) uint8
 *   [n, h/2, w/2, k].  pool: FC_POOL_MAX_2X2_S2 or FC_POOL_AVG_2X2_S2
 *   (FC_POOL_NONE -> FC_E_UNSUPPORTED).
 * Implemented: r = s = 3, stride 1, pad 1, c in {32, 64} (pad other channel
 * counts with pad_channels), k % 16 == 0 and k <= 128, n*h*w < 2^31 and
 * h*w*c*2 < 2^31 bytes (one image); others FC_E_UNSUPPORTED (FC_E_SHAPE for c or k not
 * multiples of 8).  All pointers, argmax included, 16-byte aligned. */
fc_status chain_conv_pool_winograd(const fc_half *x, const fc_half *U, const fc_half *b, fc_act act, fc_pool pool,
                                   fc_half *y, const fc_conv_shape *shape, uint8_t *argmax, void *stream);

/* ---- input preparation (BOLT notes, "Templated code generation": tensors
 *      whose channel count is not a multiple of 8 are zero-padded) ----
 * dst[o][j][i] = j < c_in ? src[o][j][i] : 0 for a tensor viewed as
 * [outer, c, inner]: NHWC activations use inner = 1 (outer = n*h*w); HWIO
 * weights use outer = r*s, inner = k.  c_out >= c_in.  No alignment needed. */
fc_status pad_channels(const fc_half *src, fc_half *dst, int64_t outer, int32_t c_in, int32_t c_out,
                       int32_t inner, void *stream);

/*
 * fc_probe_mfma -- measurement aid, not part of any chain: one block per CU,
 * waves_per_simd (1 or 2) waves per SIMD, each issuing iters x 8 independent
 * fp16 MFMAs (32x32x16, fp32 accumulate) on register operands (no memory
 * traffic), so that (launch time, FLOPs = blocks * 4 * waves_per_simd * iters
 * * 8 * 32768) gives the matrix-core rate the GPU sustains.  The first wave of
 * each block writes 4 counters to stamps[4 * block ...]: shader clock
 * (s_memtime) before and after its loop, then the 100 MHz real-time counter
 * before and after, from which the host derives the shader clock under full
 * MFMA load.  sink[block] receives one accumulator sum (keeps the work live).
 *   stamps: device, uint64 [4 * capacity], 8-byte aligned; sink: device,
 *   float [capacity]; capacity: blocks the buffers hold -- FC_E_SHAPE (and no
 *   launch) if the grid (the device's CU count) is larger; blocks (host, out):
 *   the grid size.  iters in 1 .. 2^20.
 * Enqueued on stream, asynchronous.  Returns the status only (fc_last_error
 * is not set by this call).
 */
fc_status fc_probe_mfma(int32_t waves_per_simd, int32_t iters, uint64_t *stamps, float *sink,
                        int32_t capacity, int32_t *blocks, void *stream);

/*
 * fc_probe_read -- measurement aid, not part of any chain: streams the nbytes
 * (a multiple of 16, >= 16) at buf once with 16-byte non-temporal loads,
 * consecutive threads on consecutive vectors, four independent loads in
 * flight per thread, two 256-thread blocks per CU (fewer for small buffers).
 * Timed by the caller around the launch, it gives the memory read rate the
 * GPU sustains for a stream of that size (cold: after other data evicted it).
 *   buf: device, 16-byte aligned; sink: device, uint32 [capacity] (one XOR of
 *   the data per block, keeps the loads live); blocks (host, out): the grid.
 *   FC_E_SHAPE (no launch) if the grid exceeds capacity.  Enqueued on stream,
 *   asynchronous.  Returns the status only.
 */
fc_status fc_probe_read(const void *buf, int64_t nbytes, uint32_t *sink, int32_t capacity, int32_t *blocks,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDCHAIN_H */
