/*
 * exq -- mixed-bitrate quantized linear layers on AMD Instinct MI355X (gfx950).
 *
 * The operation is a linear layer y = x * W^T whose weight W ([N][K], N
 * outputs, K inputs) is stored EXL2-style: every group of 128 consecutive
 * input channels has its own bit width from {2,3,4,5,6,8}, the widths of one
 * layer are mixed toward a target average bits-per-weight, and the groups
 * judged important are kept at higher width.  Sources: the exllamav2
 * repository report (nightvoyager.top), sections "innovations" and "key
 * design decisions" (arbitrary average bitrate, several bitrates spliced
 * inside one layer, important columns at higher bits); the promptquorum.com
 * "ExLlamaV2 explained" page, section "what is EXL2 quantization" (2/3/4/5/6/8
 * bit mixed to an average such as 2.55 bits per weight).  The weights are
 * dequantized on the fly inside the matmul kernels (the Q-GEMM of the
 * exllamav2 report's "solution philosophy"), never materialized.
 *
 * Readings fixed here because the pages give none:
 *   - one fp16 scale per (group, output column), symmetric round-to-nearest:
 *     s = fp16(max|w| / (2^(b-1) - 1)), code c = clamp(rint(w / s)) + 2^(b-1);
 *   - dequantized weight w_hat = fp16_RNE((c - 2^(b-1)) * s);
 *   - the EXQ1 bit layout below.
 *
 * EXQ1 layout (group size 128, G = K/128, widths b_g, P_g = sum_{h<g} b_h):
 *   qweight: one byte buffer of sum_g 16*N*b_g bytes, no padding.  Group g of
 *   column n owns b_g 16-byte words; word j is at byte 16*(N*P_g + j*N + n),
 *   so 64 consecutive columns read one contiguous kilobyte.  A column's
 *   dwords are numbered m = 4*j + r (r = dword in the word, little endian).
 *   Widths split into planes, low bits first: 2:[2] 3:[2,1] 4:[4] 5:[4,1]
 *   6:[4,2] 8:[8].  For code k in [0,128): u = k/4, e = k%4, e1 = e%2,
 *   e2 = e/2.  Plane 0 (width p0, dwords [0, 4*p0)): per = 8/p0; dword u/per,
 *   bit p0*(u%per) + 8*e2 + 16*e1.  Plane 1 (width p1, dwords
 *   [4*p0, 4*p0+4*p1)): with d = u/per and R = p0/p1, dword 4*p0 + d/R, bit
 *   p0*(u%per) + 16*e1 + p1*(d%R) + 8*e2.  Every field lies inside one dword.
 *   scales: fp16 [G][N] row-major, s(g, n) at g*N + n.
 *
 * Conventions for every entry point:
 *   - "device" pointers are HIP device memory on the current device; "host"
 *     pointers are ordinary host memory.  fp16 values are IEEE binary16 bit
 *     patterns (uint16_t).
 *   - streams are hipStream_t values passed as void* (NULL = null stream).
 *     Launching calls are asynchronous and never synchronize; faults inside a
 *     kernel surface at the caller's next synchronization.
 *   - arguments are validated before anything is launched; a call that
 *     fails validation launches nothing and leaves outputs untouched.
 *   - results are deterministic: the same inputs give the same bits.
 *   - exq_gemm, exq_gemm_gated, exq_dequant and exq_plan_run launch kernels
 *     only (no allocation, memset or wait), so they may be captured in a HIP
 *     graph, whose replays then read and write the buffers bound at capture.
 *     The one exception is the first call that expands a layer's quantized
 *     scales (exq_layer_create_qs below): make it before capturing.
 */
#ifndef EXQ_H
#define EXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EXQ_OK = 0,
    EXQ_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad width, non-finite input */
    EXQ_ERR_UNSUPPORTED = 2, /* a valid request the library does not implement (e.g. group size != 128) */
    EXQ_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    EXQ_ERR_OOM = 4          /* device or host allocation failed */
} exq_status;

typedef struct exq_layer* exq_layer_t;
typedef struct exq_plan* exq_plan_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* exq_status_string(exq_status s);

/* Text of the last error detected on the calling thread (static per-thread
 * buffer, "" if none). */
const char* exq_last_error(void);

/* ----------------------------------------------------------- host packer */

/* Bytes of EXQ1 qweight storage for a layer: sum_g b_g * group_size * N / 8.
 * widths: host, K/group_size entries.  Returns 0 if any argument is invalid
 * (K or N <= 0, group_size != 128, K % 128 != 0, width not in {2,3,4,5,6,8}). */
size_t exq_packed_bytes(int K, int N, int group_size, const uint8_t* widths);

/* Quantize and pack a layer on the host (offline step, multi-threaded).
 *   W           host, fp32 [N][K] row-major (nn.Linear weight layout)
 *   widths      host, uint8 [K/group_size], each in {2,3,4,5,6,8}
 *   qweight_out host, exq_packed_bytes() bytes, written completely
 *   scales_out  host, fp16 [K/group_size][N]
 * Quantizer: per (group g, column n), s = fp16_RNE(fp32(max|w|) / fp32(2^(b-1)-1))
 * with an fp32 division; code c = clamp(rint_even(fp32(w)/fp32(s)),
 * -(2^(b-1)-1), 2^(b-1)-1) + 2^(b-1); if s == 0 all codes are 2^(b-1).
 * Errors: EXQ_ERR_INVALID_ARG for bad sizes/pointers/widths, non-finite W,
 * or a scale that overflows fp16; EXQ_ERR_UNSUPPORTED for group_size != 128. */
exq_status exq_pack(const float* W, int K, int N, int group_size, const uint8_t* widths,
                    void* qweight_out, uint16_t* scales_out);

/* Quantize and pack a layer with quantized group scales (the exllamav2
 * report's 4-bit second-level scale code, section 创新之处, with a scan of
 * candidate scales by their error; the formula printed there is garbled, so
 * this is our specification).  Per column n, R[n] = fp16_RNE(max over the
 * column of |w|).  Per (group g, column n), with amax the group's max|w| and
 * qmax = 2^(b-1)-1:
 *   scale(q) = fp16_RNE(fp32(t * fp32(1/qmax))),  t = R (q+1)^2 / 256 (exact)
 *   qc = clamp(ceil(16 * sqrtf(amax / R)), 1, 16) - 1   (fp32, IEEE; 0 if R = 0)
 *   q  = qc, or qc - 1 if its codes give a strictly smaller squared error
 *        sum_i (w_i - w_hat_i)^2 (double, i ascending)
 * and the codes of exq_pack at scale(q).  Scale storage drops from 16 to 4
 * bits per (group, column) plus 16 per column.
 *   qweight_out host, exq_packed_bytes() bytes (EXQ1, as exq_pack)
 *   qscale_out  host, uint8 [K/128][N/2]: byte g*(N/2) + n/2 holds q of column n
 *               in its low nibble for even n, its high nibble for odd n
 *   ref_out     host, fp16 [N]: R
 * N must be even.  Errors as exq_pack. */
exq_status exq_pack_qs(const float* W, int K, int N, int group_size, const uint8_t* widths, void* qweight_out,
                       uint8_t* qscale_out, uint16_t* ref_out);

/* ------------------------------------------------- bit-width allocation */

/* The offline measurement and optimizer of the exllamav2 report (sections
 * 创新之处 and 关键设计决策: every candidate setting is measured once and a
 * simulated-annealing solver picks one per block to meet the bit budget).
 * Here a block is a group of 128 input channels of one linear, the
 * candidates are the widths {2,3,4,5,6,8}, and the measured error is the
 * squared weight error of this library's own quantizer (no calibration data:
 * see the design notes).
 *
 * exq_group_errors: err_out[g*6 + j] = sum over the group's N x 128 weights of
 * (w - w_hat)^2 at width {2,3,4,5,6,8}[j], w_hat = fp16_RNE((c - z) s) exactly as
 * exq_pack / exq_dequant produce it; accumulated in double, column order.
 *   W        host fp32 [N][K]; err_out host double [K/128][6]
 * Errors: INVALID_ARG (NULL, bad shape, non-finite W, a scale overflowing
 * fp16), UNSUPPORTED (group_size != 128). */
exq_status exq_group_errors(const float* W, int K, int N, int group_size, double* err_out);

/* exq_allocate_widths: choose width b_g in {2,3,4,5,6,8} for each of G groups,
 * b_g >= min_width[g], minimizing sum_g err[g][b_g] subject to
 * sum_g b_g * size[g] <= budget.  size[g] is the group's column count (its
 * bits are b_g * 128 * size[g]), so groups of several linears can share one
 * budget.  Start: the greedy of the multiple-choice knapsack on each group's
 * lower convex hull; then `iterations` simulated-annealing moves (change one
 * group; if that breaks the budget, pay for it by lowering other groups one
 * step at a time, each the cheapest per bit freed of four random ones;
 * Metropolis acceptance, geometric cooling over six decades) with a
 * SplitMix64 stream seeded by `seed`, then any budget left is spent
 * greedily.  The best state seen is kept, so the result never has more error
 * than the greedy start.  Deterministic for given inputs.
 *   err        host double [G][6], each >= 0 and finite
 *   size       host int32 [G], each >= 1
 *   min_width  host uint8 [G] or NULL (0 = no bound)
 *   widths_out host uint8 [G]; total_err_out host double or NULL
 * Errors: INVALID_ARG (NULL, G < 1, bad entries, iterations < 0, or a budget
 * below the smallest allowed cost). */
exq_status exq_allocate_widths(const double* err, const int32_t* size, int G, int64_t budget,
                               const uint8_t* min_width, uint64_t seed, int64_t iterations, uint8_t* widths_out,
                               double* total_err_out);

/* --------------------------------------------------------- device layers */

/* Describe a packed layer already resident in device memory.
 *   K, N        in/out features; K % 128 == 0, N % 16 == 0, both > 0 (else
 *               INVALID_ARG).  Every entry point serves N % 16 == 0; the
 *               64-column decode tiles (EXQ_VARIANT_DECODE64, decode plans)
 *               need N % 64 == 0 and report UNSUPPORTED otherwise.
 *   widths_host host, uint8 [K/128]; copied, the caller may free it
 *   d_qweight   device, 16-byte aligned EXQ1 words (borrowed: must outlive the handle)
 *   d_scales    device, 16-byte aligned fp16 [G][N] (borrowed)
 * The handle owns a few kilobytes of device metadata (the per-group offsets
 * and the width-sorted visiting order); it holds no scratch state, so any
 * number of streams may use it at once.  Errors: INVALID_ARG, UNSUPPORTED
 * (group_size != 128; 65536 or more 16-byte words per column, i.e.
 * sum(widths) >= 65536, which the 16-bit per-column word offsets cannot
 * address; 2 GiB or more of packed words, beyond the 32-bit buffer offsets),
 * OOM, HIP.  Every argument is checked before anything is allocated. */
exq_status exq_layer_create(int K, int N, int group_size, const uint8_t* widths_host,
                            const void* d_qweight, const void* d_scales, exq_layer_t* out);

/* A layer stored with quantized scales (exq_pack_qs): d_qscale (uint8
 * [K/128][N/2]) and d_ref (fp16 [N]) replace d_scales, both borrowed and
 * 16-byte aligned.  The decode kernels read the 4-bit codes (a quarter of the
 * scale bytes).  The prefill and dequant kernels read fp16 scales: the first
 * call that needs them (exq_gemm or exq_gemm_gated above 64 rows, or with the
 * prefill choice; exq_dequant; a prefill plan's creation) allocates the
 * expansion, 2*(K/128)*N bytes owned by the handle, fills it on that call's
 * stream and waits for it once.  A layer only ever decoded never holds it.
 * Every entry point accepts such a handle; a decode plan and a gated pair
 * need one storage kind for all their linears.  Errors as exq_layer_create. */
exq_status exq_layer_create_qs(int K, int N, int group_size, const uint8_t* widths_host, const void* d_qweight,
                               const void* d_qscale, const void* d_ref, exq_layer_t* out);

/* Release a handle and what it owns (not the borrowed buffers).  NULL is a no-op.
 * The caller must make sure no launched work still uses the handle. */
void exq_layer_destroy(exq_layer_t layer);

/* y = x * W_hat^T on `stream`.
 *   x  device, fp16 [M][K] row-major, 16-byte aligned
 *   y  device, fp16 [M][N] row-major, 16-byte aligned, must not overlap x
 *   M >= 1.  By default M <= 64 uses the decode kernel (each weight's
 *   (c - z) formed exactly in fp16 before the MFMA multiply-accumulate, the
 *   scale applied per group in fp32; one launch per 16 rows) and larger M
 *   the prefill kernel (W_hat decoded exactly into fp16 MFMA operands,
 *   activation tiles in LDS); exq_autotune / exq_set_variant can change the
 *   choice for M <= 64.  Accumulation is fp32 in both; output is fp16 RNE.
 *   A weight whose code is the zero point contributes an exact zero on
 *   every path, whatever its activation.
 * Accuracy: |y - y_ref| <= 2e-3 * sum_k |x_k * w_hat_k| + 1e-5 per output,
 * y_ref the exact (fp64) product of the fp16 inputs. */
exq_status exq_gemm(const void* x, int M, exq_layer_t layer, void* y, void* stream);

/* exq_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernel choice, results and errors as exq_gemm, and it calls no
 * hipMalloc, hipFree, allocating library routine or synchronization.  The only
 * call-time allocation of exq_gemm is the fp16 expansion of a quantized-scale
 * layer's group scales for the prefill kernel (exq_layer_create_qs); here every
 * call that needs it rewrites it, on `stream`, into a static device array of
 * 16 MiB (one per device, held until the process ends) and the prefill kernel
 * reads it there.  So 2*(K/128)*N must not exceed 16 MiB (else UNSUPPORTED,
 * before any launch).  Every call on one device shares that array: calls that
 * overlap on one device (other streams, or host threads) race and must be
 * ordered by the caller.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress, no allocation). */
exq_status exq_gemm_noalloc(const void* x, int M, exq_layer_t layer, void* y, void* stream);

/* h = SiLU(x * Wg_hat^T) (.) (x * Wu_hat^T), SiLU(t) = t / (1 + e^-t): a gate
 * and an up linear that share their input, fused with the activation between
 * them.  (The exllamav3 article, section "technical deep dive", fuses
 * matrix products and activation functions into single launches; SiLU of
 * the gate product times the up product is the activation of the Llama
 * feed-forward block, whose shapes the workloads use.)
 *   x         device, fp16 [M][K] row-major, 16-byte aligned
 *   gate, up  handles of equal K and N
 *   h         device, fp16 [M][N] row-major, 16-byte aligned, must not overlap x
 *   M >= 1.  M <= 64: one launch per 16 rows; a workgroup streams the same 64
 *   (or 16) columns of both linears and combines the two fp32 sums.  M > 64:
 *   the gate product is written to h by the prefill kernel, and the up
 *   product's epilogue reads it back (fp16) and writes SiLU(g) * u over it.
 * Accuracy, with E_g, E_u the exq_gemm bounds of the two products and
 * g_ref, u_ref their exact values:
 *   |h - h_ref| <= 1.1 E_g (|u_ref| + E_u) + |SiLU(g_ref)| E_u
 *                  + 2^-10 (|h_ref| + the terms before) + 1e-7
 * (1.1 bounds |SiLU'|; 2^-10 covers the fp32 evaluation and the fp16 output
 * rounding).  Deterministic.  Errors: INVALID_ARG (NULL, misaligned,
 * overlapping, gate and up of different shapes), UNSUPPORTED, HIP. */
exq_status exq_gemm_gated(const void* x, int M, exq_layer_t gate, exq_layer_t up, void* h, void* stream);

/* ------------------------------------------------------ per-shape tuning */

/* Kernel choices of exq_gemm for a layer at a row count M (1..64).  The
 * exllamav2 report (可复用的模式与技巧 and 关键设计决策) times its kernel
 * variants the first time a shape is seen -- 20 warmup and 200 timed runs
 * each -- keeps the one with the lowest interquartile-style mean (the mean of
 * the samples between the 5/16 and 11/16 quantiles) and caches the choice.
 *   EXQ_VARIANT_DEFAULT   decode in 16-row slices, 64-column tiles when a
 *                         slice has more than 4 rows, when N/64 >= 256, or
 *                         when N/64 >= 128 and a slice has 4 rows; else 16
 *                         (M <= 64 always takes this rule)
 *   EXQ_VARIANT_DECODE16  decode, 16-column tiles (16-row slices of x if M > 16)
 *   EXQ_VARIANT_DECODE64  decode, 64-column tiles (16-row slices of x if M > 16)
 *   EXQ_VARIANT_PREFILL   prefill kernel (M > 16 only)
 * Every choice meets exq_gemm's accuracy bound and is deterministic; two
 * choices may round differently. */
enum { EXQ_VARIANT_DEFAULT = 0, EXQ_VARIANT_DECODE16 = 1, EXQ_VARIANT_DECODE64 = 2, EXQ_VARIANT_PREFILL = 3 };

/* Mean of the samples between the 5/16 and 11/16 quantiles of n >= 1 values
 * (sorted; indices [5n/16, max(ceil(11n/16), 5n/16 + 1))).  Host; -1 on bad
 * arguments. */
double exq_trimmed_mean(const float* samples, int n);

/* Time every choice that applies at M (decode 16 and 64 columns; also prefill
 * when M > 16) on `stream` with x and y as for exq_gemm: `warmup` untimed and
 * `reps` timed runs each, one HIP event pair per run; keep the choice with the
 * lowest trimmed mean for (layer, M).  Later exq_gemm calls at this M use it.
 * y ends up holding that choice's result.  Synchronizes with `stream`.
 *   choice_out    host int or NULL: the chosen EXQ_VARIANT_*
 *   times_us_out  host float [2] (M <= 16) or [3] (M > 16) or NULL: the trimmed
 *                 means in microseconds, in variant order from DECODE16; -1
 *                 for DECODE64 when N % 64 != 0 (not a candidate then)
 * Not to be run while other work uses the layer at the same M.  Errors:
 * INVALID_ARG (NULL, M outside 1..64, warmup < 0, reps outside 1..100000,
 * misaligned or overlapping x/y), HIP, or a launch's own error. */
exq_status exq_autotune(const void* x, int M, exq_layer_t layer, void* y, void* stream, int warmup, int reps,
                        int* choice_out, float* times_us_out);

/* Set the choice for (layer, M) directly (EXQ_VARIANT_DEFAULT restores the rule).
 * Errors: INVALID_ARG (NULL, M outside 1..64, unknown variant, PREFILL at M <= 16),
 * UNSUPPORTED (DECODE64 for a layer with N % 64 != 0). */
exq_status exq_set_variant(exq_layer_t layer, int M, int variant);

/* Materialize W_hat^T: w_out device, fp16 [K][N] row-major (w_out[k*N + n]),
 * bit-exact fp16_RNE((c - 2^(b-1)) * s).  Meant for testing and inspection. */
exq_status exq_dequant(exq_layer_t layer, void* w_out, void* stream);

/* ------------------------------------------------------- batched launches */

/* Bind a list of independent linears into one launch (the pages' fused
 * kernels cut launch overhead at small batch, per the ainews.cool exllamav3
 * article, section "technical deep dive"; at large batch one launch also
 * lets the small linears fill the machine beside the large ones).
 *   count   number of linears, >= 1
 *   layers  host array of handles (borrowed; must outlive the plan)
 *   xs, ys  host arrays of device pointers, fp16 [M][K_i] and [M][N_i]
 *   M       >= 1, the same for every linear.  M <= 16: decode plan (column
 *           tiles of every linear, longest K first).  M > 16: prefill plan
 *           (256 x 256 output tiles of every linear, longest K first).
 * A plan owns a small device copy of these descriptors; buffers are bound at
 * creation, like a captured graph.  exq_plan_run computes every y_i =
 * x_i * W_i^T in one kernel launch, deterministically and to the same
 * accuracy bound as exq_gemm (its tiling, hence its summation order, may
 * differ from a single exq_gemm call).
 * Outputs must not overlap any input or each other.  Every argument of every
 * entry is checked before the first quantized-scale expansion of a prefill
 * plan is made.  Errors: INVALID_ARG, UNSUPPORTED (more than 65535 linears or
 * tiles of one linear; a decode plan entry with N % 64 != 0), OOM, HIP. */
exq_status exq_plan_create(int count, const exq_layer_t* layers, const void* const* xs,
                           const void* const* ys, int M, exq_plan_t* out);
exq_status exq_plan_run(exq_plan_t plan, void* stream);
void exq_plan_destroy(exq_plan_t plan);

/* ------------------------------------------------------------ diagnostic */

/* A plain streaming read, the practical HBM read ceiling that the decode
 * kernel's rate is compared with (it streams with the same 1 KB wave loads,
 * minus all decoding).  Workgroup w of sink_words reads the w-th of
 * sink_words equal slices of buf (the last one clipped) and stores the XOR
 * of every 32-bit word of its slice to sink[w]; the XOR of all of sink is
 * therefore the XOR of the whole buffer.
 *   buf         device, 16-byte aligned, bytes > 0 and a multiple of 16
 *   sink        device uint32 [sink_words], 4-byte aligned, written
 *   sink_words  1 .. 2^20, the number of workgroups
 * Asynchronous on `stream`.  Errors: INVALID_ARG, HIP. */
exq_status exq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EXQ_H */
