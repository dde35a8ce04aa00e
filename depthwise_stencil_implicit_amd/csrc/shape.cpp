// conv_out_shape: output sizes and strides of the canonical call.
//
// executorch PR #25084 ("Add triton::convolution and the conv routing
// framework"), description: one function computes the output layout that
// ATen's convolution returns; the op body and its shape-only twin both use
// it, so the output is allocated once and kernels only write into it.
// torch/_inductor/kernel/conv.py (conv_layout, channels_last_order): the
// output layout follows the input's memory format, channels-last meaning the
// channel dim has the smallest stride, then the last spatial dim, ..., then N.
//
// The rule, as ATen's convolution applies it: a 2-D or 3-D output is
// channels-last when x or w is channels-last-like and not also
// contiguous-like, else contiguous.  A 1-D call is run by ATen as a 2-D one
// with H = 1 after x has been made contiguous, so only the weight can make a
// 1-D output channels-last (NLC); an NLC x alone gives a contiguous output.
#include <cstring>

#include "internal.h"

namespace miconv {

int64_t out_len(int transposed, int64_t L, int64_t k, int64_t s, int64_t pb, int64_t pa, int64_t dil,
                int64_t op)
{
    if (!transposed) {
        const int64_t span = L + pb + pa - dil * (k - 1) - 1;
        if (span < 0) return 0;
        return span / s + 1;
    }
    return (L - 1) * s - pb - pa + dil * (k - 1) + op + 1;
}

// Dims listed fastest-first nest without overlap (size-1 dims skipped).
static bool nests(const conv_tensor &t, const int *order, int n)
{
    for (int i = 0; i < t.rank; ++i)
        if (t.sizes[i] == 0) return false;
    int64_t end = 0;
    for (int i = 0; i < n; ++i) {
        const int dim = order[i];
        if (t.sizes[dim] == 1) continue;
        if (t.strides[dim] <= 0 || t.strides[dim] < end) return false;
        end = t.strides[dim] * t.sizes[dim];
    }
    return true;
}

bool channels_last_like(const conv_tensor &t)
{
    const int nd = t.rank;
    if (nd < 3) return false;
    int cl[CONV_MAX_RANK], ct[CONV_MAX_RANK], n = 0;
    cl[n++] = 1;
    for (int dim = nd - 1; dim >= 2; --dim) cl[n++] = dim;
    cl[n++] = 0;
    n = 0;
    for (int dim = nd - 1; dim >= 2; --dim) ct[n++] = dim;
    ct[n++] = 1;
    ct[n++] = 0;
    return nests(t, cl, nd) && !nests(t, ct, nd);
}

void batched_out(const conv_desc &d, conv_tensor &y)
{
    std::memset(&y, 0, sizeof(y));
    const int nd = d.spatial + 2;
    y.rank = nd;
    y.dtype = d.dtype;
    y.sizes[0] = d.N;
    y.sizes[1] = d.C_out;
    for (int i = 0; i < d.spatial; ++i) y.sizes[2 + i] = d.out[i];
    const bool cl = (d.spatial >= 2 && channels_last_like(d.x)) || channels_last_like(d.w);
    int order[CONV_MAX_RANK], n = 0;
    if (cl) {
        order[n++] = 1;
        for (int dim = nd - 1; dim >= 2; --dim) order[n++] = dim;
        order[n++] = 0;
    } else {
        for (int dim = nd - 1; dim >= 0; --dim) order[n++] = dim;
    }
    int64_t acc = 1;
    for (int i = 0; i < nd; ++i) {
        y.strides[order[i]] = acc;
        acc *= y.sizes[order[i]] > 1 ? y.sizes[order[i]] : 1;
    }
}

}  // namespace miconv

extern "C" int conv_out_shape(const conv_desc *d, conv_tensor *y)
{
    if (!d || !y) return CONV_EINVAL;
    if (d->spatial < 1 || d->spatial > 3 || d->x.rank != d->spatial + 2) return CONV_EINVAL;
    conv_tensor yb;
    miconv::batched_out(*d, yb);
    if (!d->unbatched) {
        *y = yb;
        return CONV_OK;
    }
    std::memset(y, 0, sizeof(*y));
    y->rank = yb.rank - 1;
    y->dtype = yb.dtype;
    for (int i = 1; i < yb.rank; ++i) {
        y->sizes[i - 1] = yb.sizes[i];
        y->strides[i - 1] = yb.strides[i];
    }
    return CONV_OK;
}
