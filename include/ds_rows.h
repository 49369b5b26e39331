/*
 * ds_rows.h -- row-wise L2 normalisation on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Plain pointers and sizes; no HIP or
 * torch types except an opaque stream handle.  All element buffers are device
 * memory unless stated otherwise.
 *
 * Operations (cited by page and section):
 *
 *  ds_l2_rows             TensorFold PR #1260, the commit adding the two
 *                         unit-sphere row kernels of the looped nGPT model:
 *                         y = bf16(s / sqrt(sum(s^2) + eps)), s = x, or
 *                         s = bf16(x + r) with a residual (the loop entry
 *                         l2(state + input); with no residual, the loop exit).
 *  ds_slerp_rows          same commit: the nGPT residual update
 *                         h = bf16(l2(a + |alpha| (b - a))), a = bf16(l2(res)),
 *                         b = bf16(l2(out)), the lerp in fp32 steps.
 *  ds_weight_rownorm_gain DragonScale README, "What DragonScale changes":
 *                         W_eff = diag(g) r W / ||W||_row over a ragged batch of
 *                         weight matrices in one call ("Kernels and speed": the
 *                         weights of every layer in a few launches).
 *  ds_gate_l2_rows        TensorFold PR #1260, the commit adding two activation
 *  ds_swiglu_l2_rows      rows for Dory: the output gate and the scaled SwiGLU,
 *                         each rounded to bf16 and then L2-normalised over the
 *                         whole row.
 *  ds_qk_rows_l2          same PR, the q/k commit: rotate-half RoPE, each
 *                         head's L2 norm, q's scale vector (dory.py's order).
 *  ds_rms_rows            the parameter-free RMSNorm of the ternary/8-bit GPT
 *                         model page (its rms_norm over the last dimension):
 *                         y = bf16(s / sqrt(sum(s^2) / n + eps)), s as for
 *                         ds_l2_rows; ds_rms_rows_backward is its gradient.
 *  ds_rescale_project     DragonScale README, "Optimizer" (method "rescale":
 *  ds_rescale_after_step  raw rows kept at their radius by the optimizer):
 *                         remove the radial part of each gradient before a
 *                         step; after it, of the momentum, and rescale each
 *                         row to its radius.  Ragged, like the weight op.
 *  ds_l2_rows_backward    the gradient of ds_l2_rows' s -> s / sqrt(sum s^2 +
 *                         eps): ds = (dy - s <s,dy> / D^2) / D, shared by x
 *                         and r (the bf16 rounding of s passes it through).
 *  ds_weight_rownorm_gain_backward
 *                         DragonScale README, "What DragonScale changes": the
 *                         gradient reaching W is (g r / ||W||) times dL/dW_eff
 *                         with its component along the row removed; the gain's
 *                         gradient follows by the chain rule through W_eff.
 *                         Both for a ragged batch in one call.
 *  ds_weight_rownorm_gain_backward_noalloc
 *                         the same gradients for callers that cannot allocate
 *                         device memory (graph capture, serving loops): a
 *                         scalar gain's row shares in a fixed library array.
 *
 * Numerics.  bf16 values are passed as their 16-bit patterns; every rounding
 * to bf16 is to nearest, ties to even.  Sums of squares accumulate in fp32
 * (the DragonScale README's eager reference: fp32 accumulation).  eps is
 * added to the sum of squares, as an fp32 value.  The inverse length
 * 1 / sqrt(S + eps) of an activation row is computed to within 1.5 units of
 * fp32 rounding (hardware estimate plus one Newton step); a weight row's
 * length is a correctly rounded fp32 square root and its scale g * r / length
 * a correctly rounded division.  Each output is one fp32 product rounded to
 * bf16.  A row whose fp32 sum of squares would
 * overflow, or whose sum plus eps falls below 2^-96, is rescaled by a power
 * of two before summing, so every finite input row gives the float64 result
 * to within the stated rounding.  NaN and infinity propagate as in IEEE
 * arithmetic (a row holding an infinity maps its finite entries to 0 and the
 * infinity to NaN; a row holding a NaN maps to NaN).
 *
 * Gradients are those of the unrounded forward function, evaluated at the
 * forward's inputs (which the gradient calls take again: nothing is saved
 * between calls).  A gradient element is a difference of two terms that may
 * cancel; its error is within one unit of the output format's rounding plus
 * a few fp32 units of the larger term.
 *
 * Determinism.  The bits of output row i depend only on row i's inputs, cols,
 * eps (and alpha, gain, radius): not on the row count, the row's position,
 * the grid, the other matrices of a ragged call, or the stream.  Repeated
 * calls give identical bits.
 *
 * Errors.  Every argument is validated before anything is enqueued; a call
 * that returns an error has enqueued nothing.  Launch failures reported by
 * the runtime right after the launch return DS_ERR_LAUNCH.  No exception or
 * abort crosses the ABI.  Calls are thread-safe.
 *
 * Ownership.  The caller owns every device buffer and keeps it alive until
 * the stream has run the kernels.  The library keeps no caller pointer after
 * the call returns, except inside the kernels it has enqueued.
 */
#ifndef DS_ROWS_H
#define DS_ROWS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS_ROWS_VERSION 10900          /* major * 10000 + minor * 100 + patch */
#define DS_MAX_COLS 65536              /* widest row any entry point accepts */
#define DS_MAX_ELEM_COLS 16384         /* widest fp32 weight row whose width is
                                          not a multiple of 4 */
#define DS_SCRATCH_FLOATS 1048576      /* fp32 values of the fixed device scratch
                                          each GPU holds for the allocation-free
                                          entry point (4 MiB) */

/* A hipStream_t passed as an opaque pointer; NULL is the default stream. */
typedef void* ds_stream_t;

/* Status codes returned by every entry point. */
enum {
  DS_OK = 0,
  DS_ERR_NULL = -1,    /* a required pointer is NULL */
  DS_ERR_SHAPE = -2,   /* rows < 0, cols not a multiple of 8 (bf16 rows), cols
                          below 8 (bf16) or 1 (fp32 weight rows) or above
                          DS_MAX_COLS (DS_MAX_ELEM_COLS for a weight width
                          that is not a multiple of 4), or sizes that overflow */
  DS_ERR_ALIGN = -3,   /* a pointer is not 16-byte aligned (gain, norm_out and
                          dgain: 4-byte aligned) */
  DS_ERR_ARG = -4,     /* eps negative or not finite, radius not finite,
                          n < 0, or buffers that partly overlap */
  DS_ERR_ALLOC = -5,   /* the descriptor staging area could not be allocated */
  DS_ERR_LAUNCH = -6,  /* the HIP runtime reported an error for the launch,
                          the copy or the stream */
  DS_ERR_DEVICE = -7,  /* no usable HIP device */
  DS_ERR_CAPTURE = -8, /* reserved: no call returns it (a ragged weight call
                          on a capturing stream splits its launches instead;
                          see ds_weight_rownorm_gain) */
  DS_ERR_SCRATCH = -9  /* an allocation-free call needs more of the library's
                          fixed scratch than DS_SCRATCH_FLOATS */
};

/*
 * ds_l2_rows -- unit-length activation rows, optionally with a fused residual.
 * (TensorFold PR #1260, the l2 row kernel.)
 *
 *   s = x               when r == NULL
 *   s = bf16(x + r)     otherwise (the sum in fp32, rounded once to bf16)
 *   y = bf16(s / sqrt(sum_j s_j^2 + eps))          for every row
 *
 * x, r, y : row-major [rows, cols] bf16 bit patterns, contiguous, 16-byte
 *           aligned.  y may be the same buffer as x or r (each row is read
 *           whole before it is written); any other overlap is refused.
 * rows    : >= 0; 0 enqueues nothing and returns DS_OK (pointers unchecked).
 * cols    : multiple of 8, 8 <= cols <= DS_MAX_COLS.
 * eps     : finite, >= 0 (1e-6 in the pages' models).
 * stream  : the hipStream_t to launch on.
 */
int ds_l2_rows(const uint16_t* x, const uint16_t* r, uint16_t* y,
               int64_t rows, int64_t cols, float eps, ds_stream_t stream);

/*
 * ds_rms_rows -- RMS-normalised activation rows, optionally with a fused
 * residual.  (The ternary/8-bit GPT model page: its parameter-free rms_norm,
 * torch's rms_norm over the last dimension, eps 1e-6.)
 *
 *   s = x, or bf16(x + r)                          (as in ds_l2_rows)
 *   y = bf16(s / sqrt(sum_j s_j^2 / cols + eps))   for every row
 *
 * The fp32 sum of squares is divided by cols (IEEE division) before eps is
 * added; the rest is ds_l2_rows' arithmetic, rescue included.  Arguments,
 * layout, aliasing and errors: as for ds_l2_rows.
 */
int ds_rms_rows(const uint16_t* x, const uint16_t* r, uint16_t* y,
                int64_t rows, int64_t cols, float eps, ds_stream_t stream);

/*
 * ds_slerp_rows -- the nGPT residual update on unit rows.
 * (TensorFold PR #1260, the slerp row kernel.)
 *
 *   a = bf16(l2(res)),  b = bf16(l2(out))               (l2 as in ds_l2_rows)
 *   u_j = a_j + |alpha_j| * (b_j - a_j)    three fp32 operations, in this
 *                                          order, each rounded; u unrounded
 *   h = bf16(l2(u))
 *
 * res, out, h : row-major [rows, cols] bf16 bit patterns, contiguous, 16-byte
 *               aligned; h may be the same buffer as res or out.
 * alpha       : [cols] fp32, one value per column shared by all rows (the
 *               caller forms it; the kernel takes its absolute value);
 *               16-byte aligned; must not overlap h.
 * rows, cols, eps, stream : as for ds_l2_rows.
 */
int ds_slerp_rows(const uint16_t* res, const uint16_t* out, const float* alpha,
                  uint16_t* h, int64_t rows, int64_t cols, float eps,
                  ds_stream_t stream);

/*
 * ds_gate_l2_rows -- the gated attention output, unit-length per row.
 * (TensorFold PR #1260, the activation-row commit: Dory's output gate, then
 * the row's L2 norm over all its heads.)
 *
 *   t_j = bf16(o_j * sigmoid(g_j * sg_j))    g_j * sg_j one fp32 product;
 *                                            sigmoid(x) = 1 / (1 + exp(-x))
 *                                            in fp32, IEEE division
 *   y   = bf16(t / sqrt(sum_j t_j^2 + eps))
 *
 * o, g, y : row-major [rows, cols] bf16 bit patterns, contiguous, 16-byte
 *           aligned; y may be the same buffer as o or g.
 * sg      : [cols] fp32 scale vector shared by all rows (formed by the caller),
 *           16-byte aligned, not overlapping y.
 * rows, cols, eps, stream : as for ds_l2_rows.
 *
 * exp is 2^(x log2 e) on the hardware exponential with log2 e split in two
 * fp32 parts: within 1.22 ulp (measured) where the result is a normal fp32
 * number; below that it may flush, which leaves 1 + exp(-x) = 1 unchanged.  An
 * argument beyond fp32's exp range gives sigmoid 0, as fp32 arithmetic does.
 */
int ds_gate_l2_rows(const uint16_t* o, const uint16_t* g, const float* sg, uint16_t* y,
                    int64_t rows, int64_t cols, float eps, ds_stream_t stream);

/*
 * ds_swiglu_l2_rows -- the scaled SwiGLU product, unit-length per row.
 * (TensorFold PR #1260, the activation-row commit: Dory's MLP.)
 *
 *   a_j = bf16(g_j * sug_j),  b_j = bf16(u_j * suu_j)     fp32 products, rounded
 *   p_j = bf16(silu(a_j) * b_j)        silu(x) = x / (1 + exp(-x)) in fp32,
 *                                      IEEE division, exp as for the gate
 *   y   = bf16(p / sqrt(sum_j p_j^2 + eps))
 *
 * g, u, y  : row-major [rows, cols] bf16 bit patterns, contiguous, 16-byte
 *            aligned; y may be the same buffer as g or u.
 * sug, suu : [cols] fp32 scale vectors shared by all rows, 16-byte aligned,
 *            not overlapping y.
 * rows, cols, eps, stream : as for ds_l2_rows.
 */
int ds_swiglu_l2_rows(const uint16_t* g, const uint16_t* u, const float* sug, const float* suu,
                      uint16_t* y, int64_t rows, int64_t cols, float eps, ds_stream_t stream);

/*
 * ds_qk_rows_l2 -- q and k heads of a token row: RoPE, unit-length heads, q scale.
 * (TensorFold PR #1260, the q/k commit, in dory.py's order.)
 *
 * For each row (token) with position p and each head x of q and of k
 * (head_dim = HD values, halves x1 = x[0 : HD/2], x2 = x[HD/2 : HD]):
 *   t_i  = fp32(p) * inv_freq_i                            fp32 product
 *   r    = bf16([x1 cos t - x2 sin t, x2 cos t + x1 sin t])  rotate-half RoPE,
 *          each product and sum an fp32 operation; cos, sin: the device
 *          library's sincosf of the fp32 angle
 *   n    = bf16(r / sqrt(sum r^2 + eps))                    per head
 *   q_out = bf16(n * q_scale)  (one fp32 product per element); k_out = n
 *
 * q, q_out : [rows, ldq] / [rows, ldq_out] bf16 bit patterns, the first
 *            n_q_heads * head_dim elements of each row used; 16-byte aligned,
 *            strides multiples of 8.  q_out may be q itself (with ldq_out ==
 *            ldq); otherwise it must not overlap any input.
 * k, k_out : likewise for the n_kv_heads heads of k (may be NULL when
 *            n_kv_heads == 0).
 * positions: [rows] int32 token positions (converted to fp32, exact below
 *            2^24); 4-byte aligned.
 * inv_freq : [head_dim / 2] fp32 (formed by the caller, e.g. theta^(-2i/HD));
 *            16-byte aligned.
 * q_scale  : [n_q_heads * head_dim] fp32 (formed by the caller); 16-byte aligned.
 * head_dim : 128 or 256.  eps: finite, >= 0.  rows >= 0 (0: no-op).
 * The KV-cache writes that follow in a serving stack are the caller's.
 */
int ds_qk_rows_l2(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk,
                  const int32_t* positions, const float* inv_freq, const float* q_scale,
                  uint16_t* q_out, int64_t ldq_out, uint16_t* k_out, int64_t ldk_out,
                  int64_t rows, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  float eps, ds_stream_t stream);

/*
 * Gain modes of a weight matrix (DragonScale README, "Patching options": a
 * gain per row, one for the whole layer, or mode "unit" with no gain).
 */
enum {
  DS_GAIN_ROW = 0,      /* gain[i] for row i */
  DS_GAIN_SCALAR = 1,   /* gain[0] for every row */
  DS_GAIN_NONE = 2      /* no gain: W_eff = r W / ||W||; gain is ignored */
};

/*
 * One weight matrix of a ds_weight_rownorm_gain call.
 *
 * w        : [rows, cols] fp32, row-major, contiguous; 16-byte aligned when
 *            cols is a multiple of 4, else 4-byte aligned.
 * gain     : per gain_mode: [rows] fp32 (DS_GAIN_ROW), one fp32 value
 *            (DS_GAIN_SCALAR), or ignored and may be NULL (DS_GAIN_NONE);
 *            4-byte aligned.
 * radius   : the row radius r: 1 for linears and convs, sqrt(cols) for
 *            embeddings (rows of unit RMS).  Finite.
 * norm_out : [rows] fp32, receives ||W_i|| (fp32 sum of squares, fp32
 *            square root); may be NULL; 4-byte aligned.
 * w_eff    : [rows, cols] bf16 bit patterns, receives
 *            bf16(W_i * (g_i * radius / ||W_i||)); 16-byte aligned (2-byte
 *            when cols is not a multiple of 4); must not
 *            overlap w, gain or norm_out.  A zero row gives a zero row.
 * rows     : >= 0.
 * cols     : 1 <= cols <= DS_MAX_COLS.  A multiple of 4 runs on 16-byte
 *            vectors; any other width (a convolution's in * prod(kernel),
 *            such as 3 * 7 * 7 = 147) on single elements, up to
 *            DS_MAX_ELEM_COLS.  A convolution's or an embedding's weight is
 *            such a row-major matrix of its output units (or vocabulary).
 * seg, ld  : the layout.  seg = 0: contiguous rows as above.  seg > 0: a
 *            column block, for layers whose output unit is not a stored row
 *            (DragonScale README, "Supported layers": GPT-2's Conv1D stores
 *            [in, out], a ConvTranspose [in, out / groups, k...]).  The
 *            weight is A = cols / seg stored rows, ld elements apart, and
 *            row i (an output unit) is the seg values at i * seg of each
 *            stored row: element (i, a * seg + b) sits at a * ld + i * seg + b.
 *            Conv1D: seg = 1, ld = out, cols = in.  ConvTranspose, one group
 *            per descriptor: seg = prod(k), ld = (out / groups) * seg,
 *            cols = (in / groups) * seg.  Needs 1 <= seg <= 64, cols a
 *            multiple of seg, ld >= rows * seg; w_eff (and every other
 *            per-element buffer of the call) has the same layout; fp32
 *            buffers 4-byte aligned, bf16 ones 2-byte aligned.  A seg = 1
 *            block whose rows and ld are multiples of 4, with 16-byte-aligned
 *            fp32 buffers (8-byte bf16), reads W from memory once when
 *            cols <= 768 (the single-pass tile); other blocks read it twice.
 *            Results meet the same contract either way.
 */
typedef struct ds_rownorm_desc {
  const float* w;
  const float* gain;
  float radius;
  float* norm_out;
  uint16_t* w_eff;
  int64_t rows;
  int64_t cols;
  int32_t gain_mode;    /* DS_GAIN_*; 0 (a gain per row) when left zero */
  int32_t seg;          /* 0: contiguous rows; else a column block (below) */
  int64_t ld;           /* column blocks: elements between stored rows */
} ds_rownorm_desc;

/*
 * ds_weight_rownorm_gain -- unit-length weight rows times one gain per row,
 * over a ragged batch of n matrices, in one launch per row-width class.
 * (DragonScale README, "What DragonScale changes": W_eff = diag(g) r W/||W||;
 * no eps in the formula.)
 *
 * descs  : host array of n descriptors, read during the call only.  All n
 *          are validated before anything is enqueued.
 * n      : >= 0; 0 enqueues nothing.
 * stream : the hipStream_t to launch on.
 *
 * Matrices are grouped by row width; a group of at most 48 matrices travels
 * inside the kernel arguments (no copy, no allocation).  A larger group's
 * descriptors are staged in a device table through a library-owned pinned
 * buffer, kept until the stream has consumed it (an event recorded behind the
 * launches); a slot whose copy fails is returned at once.  DS_ERR_ALLOC if
 * that buffer cannot be made.  On a stream being captured into a HIP graph
 * nothing is staged: a larger group becomes several launches of at most 48
 * matrices, each carrying its table in the kernel arguments, so any call may
 * be captured (its outputs are the same, bit for bit).
 */
int ds_weight_rownorm_gain(const ds_rownorm_desc* descs, int32_t n,
                           ds_stream_t stream);

/*
 * ds_l2_rows_backward -- the gradient of ds_l2_rows.
 *
 *   s  = x, or bf16(x + r)                       (as in ds_l2_rows)
 *   D  = sqrt(sum_j s_j^2 + eps)
 *   dx = bf16((dy - s * <s, dy> / D^2) / D)       for every row
 *
 * (I - y y^T) / D with y = s / D is the Jacobian of s -> s / D; the rounding
 * of x + r to bf16 passes the gradient through, so dx is the gradient with
 * respect to x and also, when r is given, with respect to r.
 *
 * x, r, dy, dx : row-major [rows, cols] bf16 bit patterns, contiguous,
 *                16-byte aligned.  x and r are the forward call's inputs, dy
 *                the gradient reaching its output y.  dx may be the same
 *                buffer as x, r or dy; any other overlap is refused.
 * rows, cols, eps, stream : as for ds_l2_rows (eps must be the forward's).
 */
int ds_l2_rows_backward(const uint16_t* x, const uint16_t* r, const uint16_t* dy,
                        uint16_t* dx, int64_t rows, int64_t cols, float eps,
                        ds_stream_t stream);

/*
 * ds_rms_rows_backward -- the gradient of ds_rms_rows.
 *
 *   D  = sqrt(sum_j s_j^2 / cols + eps)
 *   dx = bf16((dy - s * <s, dy> / (cols * D^2)) / D)     for every row
 *
 * (I - s s^T / (cols D^2)) / D is the Jacobian of s -> s / D here.  The fp32
 * sums S and <s, dy> are each divided by cols before use.  Arguments,
 * layout, aliasing and errors: as for ds_l2_rows_backward.
 */
int ds_rms_rows_backward(const uint16_t* x, const uint16_t* r, const uint16_t* dy,
                         uint16_t* dx, int64_t rows, int64_t cols, float eps,
                         ds_stream_t stream);

/*
 * One weight matrix of a ds_weight_rownorm_gain_backward call.
 *
 * w, gain, radius, gain_mode : the forward call's inputs (as in
 *                              ds_rownorm_desc).
 * dw_eff   : [rows, cols] bf16 bit patterns, dL/dW_eff; aligned as w_eff.
 * dw       : [rows, cols] fp32, receives dL/dW; aligned as w.
 * dgain    : [rows] fp32, receives each row's share r <W_i, dW_eff_i> / ||W_i||:
 *            dL/dg_i with a gain per row; may be NULL; 4-byte aligned.  Must
 *            be NULL with DS_GAIN_NONE.
 * dgain_total : one fp32, receives dL/dg of a scalar gain, the sum of the
 *            rows' shares (added in an order fixed by rows alone); needs
 *            DS_GAIN_SCALAR and dgain (which then holds the shares; it may be
 *            NULL for an empty matrix, whose total is 0); NULL otherwise.
 * rows, cols : as in ds_rownorm_desc.
 * dw and dgain must not overlap any input or output of the call.
 */
typedef struct ds_rownorm_grad_desc {
  const float* w;
  const float* gain;
  float radius;
  const uint16_t* dw_eff;
  float* dw;
  float* dgain;
  int64_t rows;
  int64_t cols;
  int32_t gain_mode;    /* DS_GAIN_*; 0 (a gain per row) when left zero */
  float* dgain_total;
  int32_t seg;          /* as in ds_rownorm_desc */
  int64_t ld;
} ds_rownorm_grad_desc;

/*
 * ds_weight_rownorm_gain_backward -- gradients of ds_weight_rownorm_gain over
 * a ragged batch of n matrices.
 * (DragonScale README, "What DragonScale changes": the gradient reaching W is
 * tangent to its rows.)
 *
 * Per row i, with n_i = ||W_i||, P_i = <W_i, dW_eff_i> and g_i the row's
 * gain under gain_mode (1 with no gain):
 *   dw_i    = (g_i r / n_i) (dW_eff_i - W_i P_i / n_i^2)     fp32
 *   dgain_i = r P_i / n_i                                     fp32
 *   dgain_total = sum_i dgain_i                 (a scalar gain; fp32 sums)
 * A zero row (n_i = 0, scaled by the constant 0 in the forward) gets zero
 * gradients.
 *
 * descs, n, stream : as for ds_weight_rownorm_gain, including the grouping by
 *                    row width, the 48-matrix inline limit, the staged table
 *                    and the split launches under graph capture.
 */
int ds_weight_rownorm_gain_backward(const ds_rownorm_grad_desc* descs, int32_t n,
                                    ds_stream_t stream);

/*
 * ds_weight_rownorm_gain_backward_noalloc -- ds_weight_rownorm_gain_backward
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc.
 *
 * Same gradients, bit for bit, as ds_weight_rownorm_gain_backward on the same
 * descriptors, with two differences:
 *   - a DS_GAIN_SCALAR matrix's per-row shares are kept in a fixed device
 *     array the library holds per GPU (DS_SCRATCH_FLOATS fp32 values, 4 MiB,
 *     taken on the first call on a device and held until the process ends),
 *     not in a caller buffer: its descriptor's dgain must be NULL (else
 *     DS_ERR_ARG).  The scalar-gain matrices of one call may hold at most
 *     DS_SCRATCH_FLOATS rows together, else DS_ERR_SCRATCH (nothing
 *     enqueued); split larger calls;
 *   - every launch carries its matrix table in the kernel arguments (a width
 *     class of more than 48 matrices becomes several launches), so the call
 *     never stages a table and never returns DS_ERR_ALLOC.
 * The call allocates nothing (no hipMalloc, hipHostMalloc or hipFree) and
 * enqueues no memset; every share is written before it is read.
 *
 * All calls on one GPU share that GPU's scratch array: two calls whose
 * kernels may run at the same time on one GPU (different streams, no
 * ordering between them) race on it and their dgain_total values are
 * undefined.  Order such calls on one stream or with events.
 */
int ds_weight_rownorm_gain_backward_noalloc(const ds_rownorm_grad_desc* descs, int32_t n,
                                            ds_stream_t stream);

/*
 * One weight matrix of a rescale-method call.
 *
 * w      : [rows, cols] fp32 raw rows, row-major, contiguous; aligned as in
 *          ds_rownorm_desc.
 * v      : [rows, cols] fp32, the gradient (ds_rescale_project) or the
 *          momentum (ds_rescale_after_step: Adam's exp_avg, SGD's or Muon's
 *          momentum buffer; may be NULL there); updated in place; aligned
 *          as w; must not overlap any w or other v of the call.
 * radius : the row radius after a step (1 for linears and convs, sqrt(cols)
 *          for embeddings); finite.  Unused by ds_rescale_project.
 * rows, cols : as in ds_rownorm_desc.
 */
typedef struct ds_rescale_desc {
  float* w;
  float* v;
  float radius;
  int64_t rows;
  int64_t cols;
  int32_t seg;          /* as in ds_rownorm_desc */
  int64_t ld;
} ds_rescale_desc;

/*
 * ds_rescale_project -- before an optimizer step: remove from each gradient
 * row the part that would change the row's length.
 * (DragonScale README, "Optimizer".)
 *
 *   v_i <- v_i - w_i <w_i, v_i> / ||w_i||^2        fp32, per row; w read only
 *
 * A zero row of w leaves v's row unchanged.  descs, n, stream: as for
 * ds_weight_rownorm_gain (grouping by width, the 48-matrix inline limit,
 * the staged table, the split launches under graph capture).
 */
int ds_rescale_project(const ds_rescale_desc* descs, int32_t n, ds_stream_t stream);

/*
 * ds_rescale_after_step -- after an optimizer step: remove the same part from
 * the momentum, then rescale each row to its radius.
 * (DragonScale README, "Optimizer"; second moments are left alone.)
 *
 *   v_i <- v_i - w_i <w_i, v_i> / ||w_i||^2        when v is given
 *   w_i <- radius * w_i / ||w_i||                  (the stepped row's direction)
 *
 * A zero row is left as it is.  descs, n, stream: as for ds_rescale_project.
 */
int ds_rescale_after_step(const ds_rescale_desc* descs, int32_t n, ds_stream_t stream);

/* A static, human-readable string for a status code (never NULL). */
const char* ds_status_string(int status);

/* DS_ROWS_VERSION of the built library. */
int ds_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS_ROWS_H */
