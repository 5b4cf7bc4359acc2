/*
 * lb.h -- C ABI of the LittleBit factorized binary linear forward on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by short name throughout the library):
 *   [LB2 column] physicalainews.jp, "LittleBit-2: sub-1-bit LLM
 *                quantization (2026)".  Ch. 1: effective bit width of a
 *                layer, single path and residual.
 *   [LB news]    aifrontier.co.jp, "Samsung LittleBit: 13B to 0.84 GB".
 *                Sec. 2: W is approximated by two binarised (+-1) low-rank
 *                factors with FP16 row scale h, column scale g and latent
 *                scale l; a residual path is a second factorisation added
 *                at inference; inference is two small binary matrix
 *                products plus elementwise scaling.
 *
 * The layer computes, for every row x of an M x a input,
 *
 *     y = sum_p  h_p * ( S_U,p ( l_p * ( S_V,p^T ( g_p * x ) ) ) )
 *
 * with S_U,p in {+-1}^(b x s), S_V,p in {+-1}^(a x s), h_p (b), g_p (a),
 * l_p (s) in fp16, p = 0 only, or p = 0, 1 when residual.  a is the input
 * width and b the output width.  Accumulation is fp32; y is rounded once
 * to fp16 (round to nearest even).
 *
 * Conventions
 *   - Every call returns lb_status; the library never aborts or exits.
 *     lb_last_error() returns a thread-local text for the last failure.
 *   - Sign words ("canonical layout"): a factor with `rows` rows is given
 *     as rows x ceil(s/32) uint32 words, row-major; entry k of a row is
 *     bit (k % 32) of word (k / 32); bit 1 means +1 and bit 0 means -1.
 *     Bits past s are ignored.
 *   - fp16 values are passed as their IEEE binary16 bit patterns (uint16).
 *   - Host inputs are copied before the call returns; the caller may free
 *     them at once.  The library owns every device buffer it allocates.
 *   - Device pointers (x, y) are caller-owned, contiguous, row-major and
 *     16-byte aligned, and x must not overlap y.
 *   - Forward calls are asynchronous on the given hipStream_t (passed as
 *     void*, NULL = the null stream) and make no host synchronisation,
 *     with one exception each: the first call with M >= 64 on a layer
 *     builds the layer's matrix-core copy of the signs (allocates it and
 *     synchronises the device; lb_prepare does this ahead of time), and
 *     lb_stack_forward allocates (without synchronising) when M exceeds the
 *     rows reserved with lb_stack_reserve or by an earlier call, and sets
 *     up its one-launch M >= 64 path on the first call for a row count
 *     (allocates and synchronises; see lb_stack_forward).
 *   - Every buffer a forward call writes belongs to the layer or stack it
 *     runs (allocated by lb_create, lb_prepare or lb_stack_reserve) or to
 *     the caller: calls on different objects share nothing and may run on
 *     different streams at once.  Calls that use one layer or stack must be
 *     ordered on one stream: they share that object's workspace.  Nothing
 *     an object allocated is freed or moved before it is destroyed (a
 *     stack's outgrown scratch is retired, not freed).
 *   - Without a trace, lb_forward and lb_stack_forward (M within the rows
 *     already reserved, and for M >= 64 the matrix-core copies built) only
 *     launch kernels, so they can be captured into a HIP graph and
 *     replayed; such a call made under capture before that preparation
 *     returns LB_ENOTREADY instead of allocating.  The one-launch sweep
 *     carries its exchange generation from launch to launch on the device,
 *     so every replay is a fresh launch.
 */
#ifndef LB_H
#define LB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lb_layer lb_layer; /* opaque, library-owned */
typedef struct lb_stack lb_stack; /* opaque, library-owned */

typedef enum {
  LB_OK = 0,
  LB_EINVAL = -1,        /* bad argument (null pointer, size, path, overlap) */
  LB_ENOMEM = -2,        /* device or host allocation failed */
  LB_EHIP = -3,          /* a HIP runtime call failed (text in lb_last_error) */
  LB_ENOTREADY = -4,     /* forward before signs and scales of every path */
  LB_EUNSUPPORTED = -5,  /* valid request the library cannot run here */
  LB_ETIMEOUT = -6       /* a device-side wait gave up (watchdog) */
} lb_status;

/* ---------------------------------------------------------------- layers */

/* Create a layer with input width a, output width b, rank s, and one
 * path (residual = 0) or two (residual = 1), on the current HIP device.
 * [LB2 column] Ch. 1 names a, b, s and residual; [LB news] Sec. 2 the
 * structure.  a, b, s >= 1, a, b <= 2^24 and s <= 4096.  Allocates the
 * layer's device storage: the signs once (in 16-row tile layouts that
 * every kernel for M < 64 reads: about P s (a + b) / 8 bytes), the scales
 * and their tile copies, and the layer's own forward workspace (chunk
 * partials and latent rows of up to 63 rows, the matrix-core latent and
 * split-K partials, the one-row launch's state).  The matrix-core copy of
 * the signs (the same count again) is added by lb_prepare or the first
 * forward with M >= 64.  *out is set on success only. */
lb_status lb_create(int64_t a, int64_t b, int64_t s, int residual, lb_layer **out);

/* Set the sign factors of one path (0, or 1 when residual) from host
 * canonical words: su is b x ceil(s/32), sv is a x ceil(s/32).  The words
 * are re-laid out for the device and copied synchronously (the device is
 * synchronised before return, so launches on any stream see them);
 * bit-exact.  A matrix-core copy already built is rebuilt too. */
lb_status lb_pack_signs(lb_layer *L, int path, const uint32_t *su, const uint32_t *sv);

/* Set the fp16 scales of one path from host arrays: h (b values, row /
 * output scale), g (a values, column / input scale), l (s values, latent
 * scale), [LB news] Sec. 2.  Copied synchronously (as lb_pack_signs). */
lb_status lb_set_scales(lb_layer *L, int path, const uint16_t *h, const uint16_t *g,
                        const uint16_t *l);

/* y[M x b] = layer(x[M x a]); x, y are device fp16.  M = 0 is a no-op.
 * M < 64 runs the wave-level binary GEMV path (sign-flip identity on
 * packed bits, fp32 throughout): one launch for M = 1 on small layers
 * (a <= 4096 and P s <= 256, e.g. the 4096^2 projections at 0.1 bits per
 * weight; workgroups take the first product, the reduction over input
 * chunks and the second product by an atomic ticket, each waiting only on
 * workgroups that started before it, so it needs no co-residency and may
 * share the device with other streams), three launches otherwise (faster
 * for larger layers); M >= 64 runs the fp16 matrix-core
 * path (two launches: the first product with split K, then the second), in
 * which the latent vector t is rounded once to fp16 before the second
 * product; the +-g and +-l operands are exact.  The first call with
 * M >= 64 on a layer builds its matrix-core copy of the signs (allocates,
 * synchronises the device; LB_ENOTREADY instead when `stream` is being
 * captured: call lb_prepare first).  Returns LB_ENOTREADY
 * unless every path has signs and scales; LB_ETIMEOUT (running nothing)
 * when an earlier one-row forward on the device gave up a bounded
 * device-side wait (which does not happen while the device runs its work;
 * the flag is then cleared). */
lb_status lb_forward(const lb_layer *L, const void *x, void *y, int64_t M, void *stream);

/* lb_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * for M >= 2 the same kernels and the same result as lb_forward, bit for
 * bit (for M = 1 on a small layer the wave path's three launches, where
 * lb_forward takes one;
 * the two agree at the parity bar), but the scratch they need lives in one fixed 32 MB device array of the library
 * (16 KB of split-K tile counters plus 32 MB - 16 KB of workspace), held on
 * each device the library runs on until the process ends, instead of the
 * layer's own workspace.  Allocates nothing and makes no host
 * synchronisation.  The first call on a device looks the array's address
 * up (hipGetSymbolAddress) and clears its counters with a kernel on
 * `stream`; every launch leaves them zero.  All calls on one device share
 * the array, which keeps the last call's contents: calls that overlap on
 * one device (other streams, concurrent host threads) race, so order them.
 * M < 64 runs the wave path in row blocks that fit the array; M >= 64 the
 * matrix-core path, which needs its latent (256 rows of the padded latent
 * width) and split partials within the array, and the layer's matrix-core
 * copy of the signs built beforehand (lb_prepare, or an earlier lb_forward
 * with M >= 64; LB_ENOTREADY, nothing launched, otherwise).  LB_EUNSUPPORTED, with
 * nothing launched, when a layer needs more (not even one wave-path row, or
 * the matrix-core path, fits); the other errors as lb_forward. */
lb_status lb_forward_noalloc(const lb_layer *L, const void *x, void *y, int64_t M, void *stream);

/* Read the device signs of one path back into canonical words (padding
 * bits zero).  Bit-exact inverse of lb_pack_signs; synchronous. */
lb_status lb_unpack_signs(const lb_layer *L, int path, uint32_t *su, uint32_t *sv);

/* Read the fp16 scales of one path back (h: b values, g: a, l: s), the
 * bit patterns lb_set_scales or lb_init_from_factors stored; synchronous.
 * LB_ENOTREADY when that path's scales were never set. */
lb_status lb_get_scales(const lb_layer *L, int path, uint16_t *h, uint16_t *g, uint16_t *l);

/* Set the signs and scales of one path from real factors W ~= U V^T
 * (Dual-SVID, [LB news] Sec. 2): U is b x s and V is a x s, fp32,
 * row-major (row stride s), device memory on the layer's device, 4-byte
 * aligned, read on `stream` after the work already queued there and left
 * unchanged.  Readings of the one-line description, stated here:
 *   S_U = sign(U), S_V = sign(V), with sign(0) = sign(-0) = +1;
 *   |U| ~= h l_u^T and |V| ~= g l_v^T by the top singular pair of each
 *   (the best rank-1 fit in the Frobenius norm; both vectors >= 0), the
 *   singular value split evenly between the two vectors;
 *   l = l_u * l_v (elementwise), so that diag(h) S_U diag(l) S_V^T diag(g)
 *   approximates U V^T;
 *   h, g and l are rounded once to fp16 (nearest even).
 * The pair is found on the device by power iteration in fp64 with
 * fixed-order sums (deterministic), until successive unit iterates differ
 * by at most 1e-13 in every entry, within 2048 steps.  The truncated SVD
 * that gives U and V from W, and the residual W - W_1 for path 1, are the
 * caller's (e.g. a library SVD on the device).  Allocates device
 * temporaries of about 8 (s max(a, b) / 64 + a + b + 4 s) bytes plus the
 * sign words and scales, and synchronises `stream` several times; returns
 * when the layer holds the new path.  LB_EUNSUPPORTED,
 * with the layer unchanged, when the iteration has not settled (a top
 * singular value of |U| or |V| not separated from the next).
 * R, when not NULL, is an s x s fp64 row-major rotation on the device (8-byte
 * aligned, e.g. from lb_joint_itq): the path is then set from the fp64
 * factors U R and V R instead (one rocBLAS dgemm; about 16 (a + b) s more
 * bytes of device temporaries; (a + b) s < 2^31). */
lb_status lb_init_from_factors(lb_layer *L, int path, const float *U, const float *V,
                               const double *R, void *stream);

/* Joint-ITQ rotation ([LB2 column] Ch. 2): an orthogonal R between the
 * factors leaves U V^T unchanged, so LittleBit-2 rotates U <- U R and
 * V <- V R before binarising (pass R to lb_init_from_factors); R is found
 * by iterating on the stacked factors X = [U; V].  Readings, stated here:
 *   the iteration is iterative quantisation: one step sets B = sign(X R)
 *   (sign(0) = +1), then R = the orthogonal polar factor of X^T B (the
 *   orthogonal Procrustes solution, which minimises ||B - X R||_F), so the
 *   loss never increases; the pages' default is 50 steps;
 *   the start is R0 (device, s x s, fp64 row-major) or the identity when
 *   R0 is NULL.
 * U (b x s) and V (a x s) are fp32 row-major device arrays, read only; R
 * receives the s x s fp64 row-major rotation (device; may be R0).  All
 * arithmetic is fp64: the products are rocBLAS dgemm calls (atomics off,
 * reproducible), the polar factor a Newton-Schulz iteration run until
 * max |Z^T Z - I| <= 1e-12.  iters = 0 copies the start.  Needs
 * 1 <= a, b <= 2^24, 1 <= s <= 4096 and (a + b) s < 2^31.  Allocates
 * about 16 (a + b) s bytes of device temporaries, synchronises `stream`
 * and returns when R is written.  The library creates one rocBLAS handle
 * per device on first use and keeps it until the process ends; calls that
 * use it (this one and lb_init_from_factors with R) are serialised by a
 * library-wide lock.  LB_EUNSUPPORTED when X^T B is singular
 * or nearly so (the polar factor does not settle within 200 steps). */
lb_status lb_joint_itq(const float *U, const float *V, int64_t a, int64_t b, int64_t s, int iters,
                       const double *R0, double *R, void *stream);

/* Build now what forward calls of up to M rows read beyond the storage
 * lb_create made: for M >= 64 the matrix-core copy of the signs (bits
 * inverted and permuted for the fp16 operand sign flips; allocates and
 * synchronises the device).  Nothing for M < 64.  Call it before capturing
 * M >= 64 forwards into a graph or using lb_forward_noalloc with them.
 * The signs of every path must be set (LB_ENOTREADY otherwise). */
lb_status lb_prepare(lb_layer *L, int64_t M);

/* Device bytes the layer holds: *sign_bytes for its sign words (the tile
 * layouts, plus the matrix-core copy once built), *total_bytes for all of
 * its storage (signs, scales, workspace, one-row state).  Either pointer
 * may be NULL. */
lb_status lb_layer_device_bytes(const lb_layer *L, uint64_t *sign_bytes, uint64_t *total_bytes);

/* Shape queries. */
lb_status lb_layer_shape(const lb_layer *L, int64_t *a, int64_t *b, int64_t *s, int *residual);

lb_status lb_destroy(lb_layer *L);

/* ------------------------------------------------------- split stages */
/* The two halves of lb_forward, for callers that keep the latent vector
 * (the pages note that factorised K/V projections let a cache hold the
 * latent instead of the full width, [LB news] Sec. 4).
 * stage1: w[M x P*s] (fp32, device) = l_p * S_V,p^T (g_p * x), path-major
 *         (columns p*s .. p*s+s-1 belong to path p).
 * stage2: y[M x b] (fp16) = sum_p h_p * S_U,p w_p.  Any M >= 0. */
lb_status lb_forward_stage1(const lb_layer *L, const void *x, float *w, int64_t M, void *stream);
lb_status lb_forward_stage2(const lb_layer *L, const float *w, void *y, int64_t M, void *stream);

/* ---------------------------------------------------------- bit count */
/* Exact effective bits per weight of [LB2 column] Ch. 1:
 *   num_bits = P * (s*(a+b+16) + 16*(a+b)),  den = a*b,  P = 1 or 2.
 * Pure host arithmetic.  LB_EINVAL on overflow or a non-positive size. */
lb_status lb_eff_bits(int64_t a, int64_t b, int64_t s, int residual, uint64_t *num_bits,
                      uint64_t *den);

/* Largest rank s >= 0 with eff_bits(a, b, s, residual) <= bpw_num/bpw_den
 * (the same formula solved for s, floor).  LB_EINVAL when the scale
 * vectors alone exceed the budget. */
lb_status lb_rank_for_bpw(int64_t a, int64_t b, uint64_t bpw_num, uint64_t bpw_den, int residual,
                          int64_t *s);

/* -------------------------------------------------------------- stacks */
/* A stack is an ordered list of layers grouped into units: the layers of
 * one unit read the same input and have the same a and b; unit u+1 has
 * a = unit u's b.  Unit 0 reads the stack input x0.  Unit u+1 reads
 * fp16(kappa / sqrt(n_u) * sum of unit u's outputs), computed in fp32 from
 * the fp16 outputs, where n_u is unit u's layer count; the stack output
 * is the same combine of the last unit.  (The transformer parts between
 * LittleBit layers are not LittleBit layers; these linear stand-ins keep
 * the activations O(1).)  E.g. a Llama MLP stack has units [gate, up],
 * [down] per block.  Layers stay owned by the caller and must outlive the
 * stack; their signs and scales must be set before lb_stack_create.      */
lb_status lb_stack_create(lb_layer *const *layers, int n_layers, const int32_t *unit_sizes,
                          int n_units, float kappa, lb_stack **out);

/* Run the whole stack on device fp16 x0 [M x a_0] into y [M x b_last].
 * trace, when not NULL, receives every layer's fp16 output followed by
 * every unit's fp16 input, each M rows, in stack order (size from
 * lb_stack_trace_elems).  Automatic mode:
 *   M = 1       one launch for the whole sweep: one workgroup per compute
 *               unit, the latent vector of each unit summed across
 *               workgroups through device memory with bounded waits.  Its
 *               workgroups wait for one another, so all of them must be
 *               resident at once: run it while other streams' kernels do
 *               not hold the compute units.  A wait that gives up (e.g.
 *               when they do) sets a flag that lb_stack_check reports and
 *               that the next sweep returns as LB_ETIMEOUT;
 *   M = 2       without a trace: the one-launch sweep once per row (each
 *               row's output is exactly its M = 1 output);
 *   M >= 3      without a trace (M >= 2 when the device cannot hold the
 *               sweep): the whole stack in one launch per 256 rows on the
 *               matrix cores, its 32-row blocks pipelined through the units
 *               (as mode 3; measured faster than the per-layer kernels from
 *               3 rows, where the wave path has become ALU-bound).  The
 *               first such call builds the layers' matrix-core sign copies
 *               (lb_prepare, or lb_stack_reserve, does it ahead), and the
 *               first call for a row count sets up the launch's arguments
 *               (both allocate and synchronise the device).  While the
 *               stream is being captured before either exists, the
 *               per-layer kernels below run instead;
 *   otherwise   (a trace, a width that is not a multiple of 8, or that
 *               capture): for M < 64 the wave-path kernels of each layer,
 *               then a combine kernel per unit (fused into the unit's last
 *               layer up to 16 rows), or the sweep once per row for M <= 2
 *               (M <= 3 when the stack's mean matrix has at least 2^27
 *               weights) without a trace; for M >= 64 two matrix-core
 *               launches per unit, the combine fused into the second (the
 *               same tiles in the same order as the one launch, so the same
 *               output bit for bit).
 * x0, y and trace must be 16-byte aligned; y must not overlap x0. */
lb_status lb_stack_forward(lb_stack *S, const void *x0, void *y, void *trace, int64_t M,
                           void *stream);

/* Reserve the stack's scratch for up to M rows now (allocates; for
 * M >= 3, when the stack has a one-launch plan, or M >= 64, also builds
 * the layers' matrix-core sign copies, which synchronises the device), so
 * that later lb_stack_forward calls with at most M rows allocate nothing
 * except the one-launch setup of a new row count.  Scratch of an earlier, smaller
 * reservation is retired, not freed (launches already queued or captured
 * keep using it), until lb_stack_destroy. */
lb_status lb_stack_reserve(lb_stack *S, int64_t M);

/* Number of fp16 elements lb_stack_forward writes to trace for M rows. */
lb_status lb_stack_trace_elems(const lb_stack *S, int64_t M, int64_t *elems);

/* Synchronise the device and report whether any earlier persistent sweep
 * of this stack gave up a device-side wait (LB_ETIMEOUT; the stack resets
 * its synchronisation words before the next sweep).  LB_OK otherwise. */
lb_status lb_stack_check(lb_stack *S);

/* Diagnostics: record, in later persistent sweeps, eight device timestamps
 * (100 MHz counter) per phase and workgroup, taken by its first thread, into
 * the caller's device buffer buf (uint64, layout [workgroup][phase][8]:
 * phase start, second-product lookups done (first wave), second product
 * done (epilogue and combine), first-product tables built, first product done, exchange
 * level A done, level B done, exchange done).  *needed receives the element
 * count.  buf = NULL turns recording off.  The buffer must outlive its use. */
lb_status lb_stack_timeline(lb_stack *S, void *buf, int64_t capacity, int64_t *needed);

/* Diagnostics: test the failure path of the one-launch sweep.  With enable
 * != 0, later persistent sweeps of this stack wait for words nobody writes,
 * with a bound of 2048 polls, so every device-side wait gives up: the
 * kernel ends normally, its output is undefined, and lb_stack_check then
 * returns LB_ETIMEOUT.  enable = 0 restores normal sweeps.
 * LB_EUNSUPPORTED when the stack has no persistent sweep. */
lb_status lb_stack_test_wait_failure(lb_stack *S, int enable);

/* Diagnostics: stress the exchange of the one-launch sweep.  With
 * max_ticks > 0 (at most 100000), later persistent sweeps make each wave
 * wait, before each step of the cross-workgroup exchange (publishing its
 * partials, the intra-XCD sum, the cross-XCD store and poll, the final
 * poll), for a pseudo-random time drawn from seed, the sweep's generation,
 * the workgroup, the wave and the step: zero or up to max_ticks ticks of
 * 10 ns.  The output must not change (every sum has a fixed order), only
 * the time.  max_ticks = 0 turns it off.  LB_EUNSUPPORTED when the stack
 * has no persistent sweep. */
lb_status lb_stack_test_delay(lb_stack *S, uint32_t seed, uint32_t max_ticks);

/* Select the execution mode of lb_stack_forward: 0 = automatic (above),
 * 1 = every layer alone (as lb_forward) followed by a combine kernel per
 * unit, 2 = the one-launch sweep only (LB_EUNSUPPORTED unless M = 1 and
 * the device can hold one workgroup per compute unit), 3 = automatic
 * (where it takes the one launch, from 3 rows without a trace) without the
 * capture fallback.  The one launch runs the whole stack per 256 rows: the
 * matrix-core tiles of the two launches per unit, in the same order
 * (identical results), as work items dealt round robin to a grid of the
 * device's resident capacity, each waiting only for the previous step of
 * its own 32-row block, so row blocks pipeline through the units (kernels
 * on other streams that hold compute units delay it until they finish);
 * its bounded waits report a give-up as LB_ETIMEOUT from the next call, and
 * the first call for a row count sets up its launch arguments (allocates,
 * synchronises; LB_ENOTREADY under capture, where mode 0 falls back to
 * the per-layer kernels).  Mode 3 needs every width to be a multiple of 8
 * (LB_EUNSUPPORTED otherwise; mode 0 then keeps the per-layer kernels). */
lb_status lb_stack_set_mode(lb_stack *S, int mode);

lb_status lb_stack_destroy(lb_stack *S);

/* ---------------------------------------------------------- diagnostics */
const char *lb_status_str(lb_status st);
const char *lb_last_error(void);
/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LB_H */
