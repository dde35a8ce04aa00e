// conv_bind: ATen-style tensor descriptors and arguments -> the canonical call.
//
// executorch PR #25084 ("Add triton::convolution and the conv routing
// framework"), description: a binding maps every convolution overload onto
// the one canonical op, filling defaults and validating the arguments; the
// canonical op carries padding before and after each spatial dim, which ATen's
// own arguments cannot express for asymmetric or 'same' padding.
//
// torch/_inductor/kernel/conv.py, the convolution lowering: an unbatched input
// gets a leading batch dim, and per-dim argument lists shorter than the
// spatial rank are broadcast (pad_listlike).
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

namespace {

int fail(char *err, size_t err_len, const char *fmt, ...)
{
    if (err && err_len) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(err, err_len, fmt, ap);
        va_end(ap);
    }
    return CONV_EINVAL;
}

// Expand a (count, values) list into r per-dim values.
bool expand(int32_t count, const int64_t *vals, int r, int64_t dflt, int64_t out[3])
{
    for (int i = 0; i < 3; ++i) out[i] = dflt;
    if (count == 0) return true;
    if (count == 1) {
        for (int i = 0; i < r; ++i) out[i] = vals[0];
        return true;
    }
    if (count != r) return false;
    for (int i = 0; i < r; ++i) out[i] = vals[i];
    return true;
}

bool dtype_ok(int32_t dt) { return dt == CONV_F32 || dt == CONV_F16 || dt == CONV_BF16; }

bool sizes_ok(const conv_tensor *t)
{
    for (int i = 0; i < t->rank; ++i)
        if (t->sizes[i] < 0 || t->strides[i] < 0) return false;
    return true;
}

}  // namespace

extern "C" int conv_bind(const conv_tensor *x, const conv_tensor *w, const conv_tensor *b,
                         const conv_args *a, conv_desc *out, char *err, size_t err_len)
{
    if (err && err_len) err[0] = '\0';
    if (!x || !w || !a || !out) return fail(err, err_len, "conv_bind: NULL argument");
    if (w->rank < 3 || w->rank > 5)
        return fail(err, err_len, "weight must have 3 to 5 dims (1 to 3 spatial), got %d", w->rank);
    const int r = w->rank - 2;
    bool unbatched;
    if (x->rank == w->rank)
        unbatched = false;
    else if (x->rank == w->rank - 1)
        unbatched = true;
    else
        return fail(err, err_len, "input has %d dims; a %d-D convolution takes %d (batched) or %d (unbatched)",
                    x->rank, r, r + 2, r + 1);
    if (!dtype_ok(x->dtype)) return fail(err, err_len, "unsupported input dtype %d", x->dtype);
    if (w->dtype != x->dtype) return fail(err, err_len, "weight dtype differs from input dtype");
    const bool has_bias = b != nullptr && b->rank != 0;
    if (has_bias && b->dtype != x->dtype) return fail(err, err_len, "bias dtype differs from input dtype");
    if (!sizes_ok(x) || !sizes_ok(w) || (has_bias && !sizes_ok(b)))
        return fail(err, err_len, "negative size or stride");

    conv_desc d;
    std::memset(&d, 0, sizeof(d));
    d.spatial = r;
    d.transposed = a->transposed ? 1 : 0;
    d.unbatched = unbatched ? 1 : 0;
    d.dtype = x->dtype;
    d.has_bias = has_bias ? 1 : 0;

    // Batched view of x.
    conv_tensor xb;
    std::memset(&xb, 0, sizeof(xb));
    xb.rank = r + 2;
    xb.dtype = x->dtype;
    if (unbatched) {
        int64_t extent = 1;
        for (int i = 0; i < x->rank; ++i)
            if (x->sizes[i] > 0) extent += (x->sizes[i] - 1) * x->strides[i];
        xb.sizes[0] = 1;
        xb.strides[0] = extent;
        for (int i = 0; i < x->rank; ++i) {
            xb.sizes[i + 1] = x->sizes[i];
            xb.strides[i + 1] = x->strides[i];
        }
    } else {
        xb = *x;
    }
    d.x = xb;
    d.w = *w;
    if (has_bias) d.b = *b;

    const int64_t groups = a->groups == 0 ? 1 : a->groups;
    if (groups < 1) return fail(err, err_len, "groups must be positive, got %lld", (long long)groups);
    d.groups = groups;
    d.N = xb.sizes[0];
    d.C_in = xb.sizes[1];
    for (int i = 0; i < 3; ++i) {
        d.in[i] = i < r ? xb.sizes[2 + i] : 1;
        d.k[i] = i < r ? w->sizes[2 + i] : 1;
    }
    for (int i = 0; i < r; ++i) {
        if (d.in[i] < 1) return fail(err, err_len, "spatial dim %d of the input is empty", i);
        if (d.k[i] < 1) return fail(err, err_len, "kernel size must be positive in dim %d", i);
    }
    if (d.C_in % groups) return fail(err, err_len, "input channels %lld not divisible by groups %lld",
                                     (long long)d.C_in, (long long)groups);
    if (!d.transposed) {
        d.C_out = w->sizes[0];
        if (d.C_out % groups) return fail(err, err_len, "output channels %lld not divisible by groups %lld",
                                          (long long)d.C_out, (long long)groups);
        if (w->sizes[1] != d.C_in / groups)
            return fail(err, err_len, "weight dim 1 is %lld, expected C_in/groups = %lld",
                        (long long)w->sizes[1], (long long)(d.C_in / groups));
    } else {
        if (w->sizes[0] != d.C_in)
            return fail(err, err_len, "transposed weight dim 0 is %lld, expected C_in = %lld",
                        (long long)w->sizes[0], (long long)d.C_in);
        d.C_out = w->sizes[1] * groups;
    }
    if (has_bias && (b->rank != 1 || b->sizes[0] != d.C_out))
        return fail(err, err_len, "bias must be [C_out] = [%lld]", (long long)d.C_out);

    int64_t st[3], pb[3], pa[3], dil[3], op[3];
    if (!expand(a->n_stride, a->stride, r, 1, st)) return fail(err, err_len, "stride needs 1 or %d values", r);
    if (!expand(a->n_dilation, a->dilation, r, 1, dil)) return fail(err, err_len, "dilation needs 1 or %d values", r);
    if (!expand(a->n_output_padding, a->output_padding, r, 0, op))
        return fail(err, err_len, "output_padding needs 1 or %d values", r);
    if (a->padding_mode == CONV_PAD_EXPLICIT) {
        if (!expand(a->n_padding, a->padding_before, r, 0, pb) ||
            !expand(a->n_padding, a->padding_after, r, 0, pa))
            return fail(err, err_len, "padding needs 1 or %d values", r);
    } else if (a->padding_mode == CONV_PAD_SAME || a->padding_mode == CONV_PAD_VALID) {
        if (a->n_padding != 0) return fail(err, err_len, "'same'/'valid' padding takes no explicit values");
        if (d.transposed) return fail(err, err_len, "'same'/'valid' padding is only defined for forward calls");
        for (int i = 0; i < 3; ++i) pb[i] = pa[i] = 0;
    } else {
        return fail(err, err_len, "unknown padding mode %d", a->padding_mode);
    }
    for (int i = 0; i < r; ++i) {
        if (st[i] < 1) return fail(err, err_len, "stride must be positive");
        if (dil[i] < 1) return fail(err, err_len, "dilation must be positive");
    }
    if (a->padding_mode == CONV_PAD_SAME) {
        for (int i = 0; i < r; ++i) {
            if (st[i] != 1) return fail(err, err_len, "'same' padding needs stride 1");
            const int64_t total = dil[i] * (d.k[i] - 1);
            pb[i] = total / 2;
            pa[i] = total - pb[i];
        }
    }
    for (int i = 0; i < r; ++i) {
        if (pb[i] < 0 || pa[i] < 0) return fail(err, err_len, "padding must be non-negative");
        if (op[i] < 0) return fail(err, err_len, "output_padding must be non-negative");
        if (!d.transposed && op[i] != 0) return fail(err, err_len, "output_padding needs a transposed convolution");
        if (d.transposed && op[i] >= (st[i] > dil[i] ? st[i] : dil[i]))
            return fail(err, err_len, "output_padding must be smaller than stride or dilation");
    }
    for (int i = 0; i < 3; ++i) {
        d.stride[i] = st[i];
        d.padding_before[i] = pb[i];
        d.padding_after[i] = pa[i];
        d.dilation[i] = dil[i];
        d.output_padding[i] = op[i];
        d.out[i] = 1;
    }
    for (int i = 0; i < r; ++i) {
        const int64_t o = miconv::out_len(d.transposed, d.in[i], d.k[i], st[i], pb[i], pa[i], dil[i], op[i]);
        if (o < 1) return fail(err, err_len, "output length in dim %d would be %lld (< 1)", i, (long long)o);
        d.out[i] = o;
    }
    *out = d;
    return CONV_OK;
}
