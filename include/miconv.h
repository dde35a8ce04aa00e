/*
 * miconv.h -- C ABI of the MI355X (gfx950) canonical convolution library.
 *
 * One canonical convolution op (executorch PR #25084, "Add triton::convolution
 * and the conv routing framework", description): explicit padding_before and
 * padding_after per spatial dim, stride, dilation, groups, and separately
 * defined forward and transposed semantics.
 *
 *   forward     y[n, g*Cog+j, o] = b[g*Cog+j]
 *                 + sum_{c<Cig} sum_t x[n, g*Cig+c, o*s - pb + t*dil] * w[g*Cog+j, c, t]
 *   transposed  y[n, g*Cog+j, o] = b[g*Cog+j]
 *                 + sum_{c<Cig} sum_t x[n, g*Cig+c, (o + pb - t*dil)/s] * w[g*Cig+c, j, t]
 *               where a term exists only when the quotient is an exact integer
 *               inside the input (executorch PR #25091, "Run transposed
 *               convolutions on the implicit-GEMM template", description: the
 *               transposed gather, with the [C_in, C_out/groups, k...] weight
 *               read with its first two axes swapped).
 *   Terms whose input index falls outside [0, L) are zero padding (the masked
 *   loads of the LOOP_BODY_2D template in torch/_inductor/kernel/conv.py).
 *
 * Four calls make up the path (the binding, the shared output layout, the
 * planner and the launch that the PR #25084 description lists):
 *   conv_bind      tensor descriptors + user arguments -> canonical conv_desc
 *   conv_out_shape conv_desc -> output sizes and strides
 *   conv_plan      conv_desc + output descriptor -> kernel choice and launch
 *   conv_run       plan + device pointers + stream -> asynchronous launch
 *
 * Conventions
 *   - Strides are in elements, not bytes.  Sizes are logical: x is
 *     [N, C_in, L_1..L_r] whatever its memory order; r = 1..3.  An unbatched x
 *     ([C_in, L...]) is accepted and gives an unbatched y.
 *   - x, w, b and y share one dtype.  Accumulation is fp32; the bias is
 *     added in fp32 and the result rounded once (nearest even) to the dtype.
 *   - The library never allocates device memory: the caller owns every
 *     buffer, the workspace and the stream.  Its only mutable global state
 *     is the cache of timed schedules (conv_tune), guarded by a mutex.
 *     conv_desc and conv_plan_t are plain caller-owned structs (no destroy
 *     call); a plan may be reused for any call with the same descriptors.
 *   - Every function is reentrant.  conv_run does not synchronise.
 */
#ifndef MICONV_H
#define MICONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MICONV_API __attribute__((visibility("default")))
#else
#define MICONV_API
#endif

#define CONV_MAX_RANK 5
#define CONV_MAX_SPATIAL 3

typedef enum conv_dtype { CONV_F32 = 0, CONV_F16 = 1, CONV_BF16 = 2 } conv_dtype;

typedef enum conv_status {
    CONV_OK = 0,
    CONV_EINVAL = 1,       /* arguments violate the op's rules */
    CONV_EUNSUPPORTED = 2, /* forced kernel outside its supported domain */
    CONV_ELAYOUT = 3,      /* y's sizes/strides differ from conv_out_shape */
    CONV_EALIGN = 4,       /* a pointer is not aligned to its element size */
    CONV_EDEVICE = 5,      /* no usable GPU, or a HIP launch/runtime error */
    CONV_ENOSPACE = 6      /* conv_run_noalloc: the plan needs more scratch than the fixed array */
} conv_status;

typedef enum conv_padding_mode {
    CONV_PAD_EXPLICIT = 0, /* padding_before / padding_after as given */
    CONV_PAD_SAME = 1,     /* stride 1 only: total dil*(k-1), before = total/2 */
    CONV_PAD_VALID = 2     /* no padding */
} conv_padding_mode;

/* Kernels the planner can choose (also the values accepted by force_kernel). */
typedef enum conv_kernel {
    CONV_K_AUTO = -1,
    CONV_K_DW_CL = 1,   /* depthwise, channel-contiguous input: per-lane register sliding window */
    CONV_K_PLANE = 2,   /* depthwise / few-channel grouped, any layout: LDS halo tile, fan-out */
    CONV_K_GRP = 3,     /* few-channel grouped, half types: packed dot2 over input-channel pairs, or
                           (plan variant 1) small 3x3 groups with contiguous planes as a per-group
                           matrix-core contraction over (tap, channel) */
    CONV_K_REDUCE = 4,  /* depthwise / few-channel grouped, few outputs: wavefront reduction over taps */
    CONV_K_IGEMM = 5,   /* implicit GEMM, forward: on-the-fly im2col tile in LDS, MFMA */
    CONV_K_IGEMM_T = 6  /* implicit GEMM with the transposed gather, phase-split by stride */
} conv_kernel;

/* A tensor descriptor: no data pointer, only shape, strides and dtype. */
typedef struct conv_tensor {
    int32_t rank;                     /* number of dims (0 = absent) */
    int32_t dtype;                    /* conv_dtype */
    int64_t sizes[CONV_MAX_RANK];
    int64_t strides[CONV_MAX_RANK];   /* elements; entries >= rank are ignored */
} conv_tensor;

/* User-level arguments, ATen style.  Each per-dimension list has a count:
 * 0 = use the default (stride 1, padding 0, dilation 1, output_padding 0),
 * 1 = broadcast the single value to every spatial dim, r = one per dim. */
typedef struct conv_args {
    int32_t transposed;               /* 0 forward, 1 transposed */
    int32_t padding_mode;             /* conv_padding_mode */
    int64_t groups;                   /* 0 = default 1 */
    int32_t n_stride, n_padding, n_dilation, n_output_padding;
    int64_t stride[CONV_MAX_SPATIAL];
    int64_t padding_before[CONV_MAX_SPATIAL];
    int64_t padding_after[CONV_MAX_SPATIAL];   /* shares n_padding */
    int64_t dilation[CONV_MAX_SPATIAL];
    int64_t output_padding[CONV_MAX_SPATIAL];
} conv_args;

/* The canonical call.  Spatial arrays hold r entries; the rest are 1 (sizes,
 * stride, dilation) or 0 (paddings).  x is the batched view of the caller's x
 * (a leading size-1 dim is added when unbatched); b has rank 0 when absent. */
typedef struct conv_desc {
    int32_t spatial;                  /* r = 1..3 */
    int32_t transposed;
    int32_t unbatched;
    int32_t dtype;
    int32_t has_bias;
    int32_t reserved0;
    int64_t N, C_in, C_out, groups;
    int64_t in[CONV_MAX_SPATIAL];
    int64_t k[CONV_MAX_SPATIAL];
    int64_t out[CONV_MAX_SPATIAL];
    int64_t stride[CONV_MAX_SPATIAL];
    int64_t padding_before[CONV_MAX_SPATIAL];
    int64_t padding_after[CONV_MAX_SPATIAL];
    int64_t dilation[CONV_MAX_SPATIAL];
    int64_t output_padding[CONV_MAX_SPATIAL];
    conv_tensor x, w, b;
} conv_desc;

/* Plan flags.  CONV_PLAN_ONE_BY_ONE: a forward 1x1 call with stride 1 and no
 * padding on dense channels-last x and a contiguous [C_out, C_in] weight
 * (C_in a multiple of 64): a plain GEMM on the implicit GEMM's tiles whose A
 * rows are x's rows and whose B operand is the weight tensor in place (no
 * position arithmetic, no weight repack). */
#define CONV_PLAN_ONE_BY_ONE 1
/* Set by conv_plan_tuned on a plan that comes from the cache of conv_tune. */
#define CONV_PLAN_TUNED 2

/* A launch plan.  Produced by conv_plan on the host without any device call. */
typedef struct conv_plan_t {
    conv_desc d;
    conv_tensor y;                    /* batched view of y */
    int32_t kernel;                   /* conv_kernel */
    int32_t variant;                  /* kernel-specific schedule id */
    int32_t vec_ok;                   /* strides allow 16-byte vector access */
    int32_t index64;                  /* some element offset needs 64 bits */
    int64_t workspace_bytes;          /* device scratch conv_run needs (0 = none) */
    int64_t tile[8];                  /* kernel-specific tile parameters */
    int64_t grid[3];
    int32_t block;
    int32_t lds_bytes;
    int32_t flags;                    /* CONV_PLAN_* bits */
    int32_t batch_chunk;              /* 0: one launch covers the batch; else images per launch (x or y
                                         spans 2 GiB or more: the kernels take 32-bit buffer offsets, so
                                         conv_run runs the batch in chunks; d and y stay the whole call,
                                         tile / grid / variant are those of a chunk) */
    int64_t flops;                    /* algorithmic FLOPs of the call */
    int64_t bytes;                    /* algorithmic bytes: x + w + b read once, y written once */
} conv_plan_t;

/*
 * conv_bind -- map tensor descriptors and ATen-style arguments onto the
 * canonical op, filling defaults and validating (executorch PR #25084,
 * description: the binding maps every convolution overload onto the
 * canonical op, filling defaults and validating the arguments).
 *
 *   x  [N, C_in, L...] or unbatched [C_in, L...]; r = rank - 2 (or - 1).
 *   w  forward [C_out, C_in/groups, k...]; transposed [C_in, C_out/groups, k...].
 *   b  [C_out] or NULL.
 *   a  user arguments (see conv_args).  'same' needs stride 1 and splits the
 *      total dil*(k-1) as before = total/2, after = total - before.
 *   out  receives the canonical call.
 *   err, err_len  optional buffer for a message on failure (may be NULL).
 *
 * Returns CONV_OK or CONV_EINVAL (rank outside 3..5 / 2..4, dtype mismatch,
 * channel or group mismatch, non-positive stride/dilation/groups, negative
 * padding, output_padding >= max(stride, dilation) or nonzero on a forward
 * call, an output length < 1, a negative size or stride).
 */
MICONV_API int conv_bind(const conv_tensor *x, const conv_tensor *w, const conv_tensor *b,
              const conv_args *a, conv_desc *out, char *err, size_t err_len);

/*
 * conv_out_shape -- the output layout, shared by the op and its planner so
 * the output is allocated once and kernels only write into it (executorch
 * PR #25084, description: the output layout ATen's convolution returns).
 *
 *   Sizes: forward O = floor((L + pb + pa - dil*(k-1) - 1)/s) + 1,
 *          transposed O = (L-1)*s - pb - pa + dil*(k-1) + op + 1.
 *   Strides: dense; channels-last (C fastest, then the last spatial dim, ...,
 *   then N) when x or w is channels-last-like and not also contiguous-like,
 *   contiguous otherwise.  Unbatched calls give an unbatched y.
 *
 * Returns CONV_OK, or CONV_EINVAL for a NULL or inconsistent descriptor.
 */
MICONV_API int conv_out_shape(const conv_desc *d, conv_tensor *y);

/*
 * conv_plan -- route the call and fix the launch (executorch PR #25084,
 * description: templates declare what they support and the planner routes
 * every overload; PR #25085, description: depthwise and up-to-8-channel
 * grouped 2-D convolutions with dilation 1 and kernels up to 9x9 go to the
 * direct stencil; PR #25091, description: transposed calls run on the
 * implicit GEMM with the transposed gather).  Host only, deterministic.
 *
 *   d            canonical call from conv_bind.
 *   y            output descriptor; must equal conv_out_shape(d) exactly.
 *   force_kernel CONV_K_AUTO, or a conv_kernel to run (tests pin schedules).
 *   p            receives the plan.
 *   Same as conv_plan_ex with { force_kernel, -1 }.
 *
 * Returns CONV_OK, CONV_ELAYOUT (y differs from conv_out_shape),
 * CONV_EUNSUPPORTED (forced kernel outside its domain) or CONV_EINVAL.
 */
MICONV_API int conv_plan(const conv_desc *d, const conv_tensor *y, int32_t force_kernel, conv_plan_t *p);

/* Options of conv_plan_ex.  Zero-initialise, then set what is wanted. */
typedef struct conv_plan_opts {
    int32_t force_kernel;             /* CONV_K_AUTO (-1) or a conv_kernel to run */
    int32_t force_variant;            /* -1 = the planner's schedule; else a schedule of the forced
                                         kernel: CONV_K_IGEMM / CONV_K_IGEMM_T take an index of the
                                         implicit GEMM's tile table (0..11 for 16-bit types except
                                         5, which is the fp32 one), CONV_K_GRP takes 0 (packed dot2)
                                         or 1 (matrix-core plane) */
    int32_t reserved[6];              /* must be zero */
} conv_plan_opts;

/*
 * conv_plan_ex -- conv_plan with explicit options: the forced kernel and,
 * for a forced kernel, one of its schedules (executorch PR #25084,
 * description: tests pin a single schedule of a template).  The planner
 * reads no environment; these fields are the only overrides.
 *
 *   o  NULL = { CONV_K_AUTO, -1 } (the same plan as conv_plan).
 *
 * Returns as conv_plan; CONV_EUNSUPPORTED also when the forced schedule
 * cannot run the call (a tile of another dtype class, the matrix-core
 * grouped schedule outside its conditions), CONV_EINVAL when a schedule is
 * given without a kernel that has schedules.
 */
MICONV_API int conv_plan_ex(const conv_desc *d, const conv_tensor *y, const conv_plan_opts *o, conv_plan_t *p);

/*
 * conv_run -- launch the planned kernels on the caller's HIP stream.
 *
 *   x, w, y      device pointers laid out as the plan's descriptors say.
 *   b            device pointer or NULL (must be non-NULL iff d.has_bias).
 *   workspace    device scratch of at least p->workspace_bytes bytes, 256-byte
 *                aligned, or NULL when p->workspace_bytes == 0.  Its content
 *                is overwritten; calls sharing one workspace must not overlap.
 *   stream       hipStream_t (NULL = the default stream).
 *
 * Asynchronous: returns after enqueueing.  A call with an empty output is a
 * no-op returning CONV_OK.  Returns CONV_EINVAL (NULL pointer, missing
 * workspace), CONV_EALIGN (a pointer not aligned to its element size) or
 * CONV_EDEVICE (no GPU, or a launch error).  16-byte vector paths are used
 * only when the pointers allow them; otherwise the scalar path of the same
 * kernel runs.
 */
MICONV_API int conv_run(const conv_plan_t *p, const void *x, const void *w, const void *b, void *y,
             void *workspace, size_t workspace_bytes, void *stream);

/* A plan of the gradients of one call (conv_plan_backward).  Caller-owned,
 * no destroy call; host-only to produce. */
typedef struct conv_bwd_plan_t {
    conv_desc d;                      /* the call whose gradients are computed */
    conv_tensor gy;                   /* batched view of the output gradient */
    conv_tensor dx;                   /* batched input gradient (layout of conv_backward_layout) */
    conv_tensor dw;                   /* weight gradient: w's sizes, dense in w's memory format */
    conv_tensor db;                   /* [C_out] contiguous, or rank 0 */
    int32_t need_dx, need_dw, need_db;
    int32_t dgrad_flip;               /* 1: dgrad reads the weight reversed from the workspace (below) */
    conv_plan_t dgrad;                /* the call that computes dx */
    int64_t wg_tile[8];               /* weight-gradient schedule */
    int64_t db_splits;                /* ranges of positions of the bias gradient */
    int64_t workspace_bytes;          /* device scratch conv_run_backward needs */
    int64_t flops[3];                 /* algorithmic FLOPs of dx, dw, db */
    int64_t bytes[3];                 /* algorithmic bytes of dx, dw, db */
} conv_bwd_plan_t;

/*
 * conv_backward_layout -- layouts of the gradients of a call
 * (torch/_inductor/kernel/conv.py, convolution_backward: the input, weight
 * and bias gradients of the convolution).
 *
 *   d   the call (conv_bind).
 *   gy  descriptor of the output gradient: y's sizes (batched, or unbatched
 *       for an unbatched call), any non-negative strides.
 *   dx  receives the input gradient's layout: the output layout of the
 *       adjoint call (forward and transposed exchanged, gy as its input, the
 *       same weight tensor), which has x's sizes.  A 16-bit channel-major gy
 *       of 16 MiB or more (each (image, channel) plane dense, C_out >= 64 and
 *       a multiple of 8) beside channels-last x is read through a
 *       channels-last copy (conv_bwd_plan_t.wg_tile[6] bytes at the start of
 *       the workspace), and dx is then the adjoint call's output on that
 *       copy (channels-last for 2-D and 3-D calls).  May be NULL.
 *   dw  receives w's sizes, dense in w's memory format.  May be NULL.
 *   db  receives [C_out], stride 1.  May be NULL.
 *
 * Returns CONV_OK, CONV_EINVAL, CONV_ELAYOUT (gy's sizes or dtype differ
 * from y's) or CONV_EUNSUPPORTED (a transposed call with output_padding >=
 * stride, whose adjoint is longer than x).
 */
MICONV_API int conv_backward_layout(const conv_desc *d, const conv_tensor *gy, conv_tensor *dx, conv_tensor *dw,
                                    conv_tensor *db);

/*
 * conv_plan_backward -- plan the gradients of a call (same passage).
 *
 *   dx = the adjoint call of gy: for a forward call the transposed call
 *        with output_padding (L + pb + pa - dil(k-1) - 1) mod s, for a
 *        transposed call the forward call; planned by conv_plan.  A forward
 *        call of stride 1 with at most 8 output channels per group (r <= 2)
 *        instead gets dgrad = the forward call of gy with padding
 *        ((k-1)dil - pb, (k-1)dil - pa) on the weight reversed along every
 *        tap dim with its two channel dims exchanged per group, a contiguous
 *        [C_in][C_out/groups][k...] copy that conv_run_backward writes at the
 *        start of the workspace (dgrad_flip = 1), when conv_plan sends that
 *        call to a stencil kernel.
 *   dw[g*PC + a, b, t] = sum over positions m of P[m, g*PC + a] *
 *        Q[m*s - pb + t*dil, g*QC + b] with (P, Q) = (gy, x) for a forward
 *        call and (x, gy) for a transposed one.
 *   db[co] = sum of gy over images and positions.
 *   need_dx / need_dw / need_db select the gradients.  Host only.
 *
 * Returns as conv_backward_layout, or CONV_EUNSUPPORTED when the adjoint
 * call cannot be planned.
 */
MICONV_API int conv_plan_backward(const conv_desc *d, const conv_tensor *gy, int32_t need_dx, int32_t need_dw,
                                  int32_t need_db, conv_bwd_plan_t *p);

/*
 * conv_run_backward -- enqueue the planned gradients on the caller's stream.
 *
 *   x, w, gy         device pointers as the plan's descriptors say (x is
 *                    needed for dw, w for dx).
 *   dx, dw, db       device outputs at the layouts of conv_backward_layout
 *                    (NULL for a gradient the plan does not compute).
 *   workspace        device scratch of at least p->workspace_bytes bytes,
 *                    16-byte aligned (NULL when 0).  Overwritten.
 *
 * Each gradient is accumulated in fp32 and rounded once.  Asynchronous.
 * Returns CONV_OK, CONV_EINVAL (a NULL pointer the plan needs, a short
 * workspace), CONV_EALIGN or CONV_EDEVICE.
 */
MICONV_API int conv_run_backward(const conv_bwd_plan_t *p, const void *x, const void *w, const void *gy, void *dx,
                                 void *dw, void *db, void *workspace, size_t workspace_bytes, void *stream);

/*
 * conv_plan_candidates -- every plan that can run a call: the rule's plan
 * first, then each kernel whose supports() holds and each schedule of the
 * kernels that have several (the implicit GEMM's tile table, the grouped
 * stencil's schedules, the transposed both-phases kernels), as conv_plan_ex
 * accepts them -- except implicit-GEMM plans that pad each group's input
 * channels more than fourfold, which multiply mostly zeros, and the generic
 * channels-last depthwise schedule where a ring schedule applies, whose
 * re-reads of input rows from L2 time well only on warm buffers (executorch PR
 * #25085, description: the stencil's schedules
 * are timed when the call is compiled; torch/_inductor/kernel/conv.py,
 * autotune_select_algorithm).  Host only.
 *
 *   out, max   caller array of max plans (may be NULL when max is 0).
 *   count      receives the number of candidates (may exceed max).
 *
 * Returns as conv_plan.
 */
MICONV_API int conv_plan_candidates(const conv_desc *d, const conv_tensor *y, conv_plan_t *out, int32_t max,
                                    int32_t *count);

/*
 * conv_tune -- time the candidates on the caller's buffers and stream and
 * keep the fastest (same passages).
 *
 *   x, w, b, yptr    device buffers of the call (y is overwritten).
 *   workspace        device scratch; candidates needing more than
 *                    workspace_bytes are skipped.
 *   reps             timed launches per candidate (after one untimed one).
 *   best             receives the fastest plan.
 *
 * The choice is cached per (descriptors, y, device) for conv_plan_tuned.
 * Synchronises the stream.  Returns CONV_OK, the planning errors of
 * conv_plan, or CONV_EDEVICE (no candidate ran).
 */
MICONV_API int conv_tune(const conv_desc *d, const conv_tensor *y, const void *x, const void *w, const void *b,
                         void *yptr, void *workspace, size_t workspace_bytes, void *stream, int32_t reps,
                         conv_plan_t *best);

/*
 * conv_plan_tuned -- the plan conv_tune chose for these descriptors on the
 * current device (flag CONV_PLAN_TUNED set), or conv_plan's when the call
 * has not been tuned.  Returns as conv_plan.
 */
MICONV_API int conv_plan_tuned(const conv_desc *d, const conv_tensor *y, conv_plan_t *p);

/* Size of the device-resident scratch array of conv_run_noalloc, MiB. */
#define MICONV_NOALLOC_SCRATCH_MIB 32

/*
 * conv_run_noalloc -- conv_run for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels, with the workspace taken from a
 * file-scope device array of MICONV_NOALLOC_SCRATCH_MIB MiB that each GPU
 * holds until the process ends.  It calls no allocating routine.
 *
 *   p, x, w, b, y, stream   as for conv_run.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: calls that overlap in time on one GPU race.  Plans whose
 * kernels need no workspace run exactly as with conv_run.
 *
 * Returns as conv_run, or CONV_ENOSPACE when p->workspace_bytes exceeds the
 * array (nothing is launched).
 */
MICONV_API int conv_run_noalloc(const conv_plan_t *p, const void *x, const void *w, const void *b, void *y,
                                void *stream);

/* Name of a conv_kernel value ("dw_cl", "plane", ...), or "?" . */
MICONV_API const char *conv_kernel_name(int32_t kernel);

/* Message for a conv_status value. */
MICONV_API const char *conv_status_string(int32_t status);

/* Library ABI version (sizes of the structs above are part of it). */
MICONV_API int32_t conv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MICONV_H */
