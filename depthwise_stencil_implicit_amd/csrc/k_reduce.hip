// Depthwise / few-channel grouped stencil for calls with few output positions
// (kernel CONV_K_REDUCE).
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: a schedule
// that reduces over the taps in parallel, for calls with few outputs.
//
// Layout on gfx950: when a call has only a handful of output positions per
// channel (a large kernel over a small input), one thread per output would
// leave most lanes idle while each walks a long tap loop.  Here one wave owns
// one output element: its 64 lanes split the Cig*KH*KW (input channel, tap)
// terms, each lane accumulates its share in fp32, and a butterfly of
// cross-lane exchanges sums the 64 partial sums.  Any memory layout.
#include "dev_common.h"
#include "internal.h"

namespace miconv {

struct RdArgs {
    const void *x, *w, *b;
    void *y;
    int64_t xs_n, xs_c, xs_h, xs_w;
    int64_t ys_n, ys_c, ys_h, ys_w;
    int64_t ws0, ws1, ws2, ws3;
    int64_t count;  // output elements
    int32_t G, Cig, Cog, C_out, H, W, OH, OW, KH, KW, SH, SW, PH, PW, DH, DW;
    int32_t has_bias;
};

template <typename T>
__global__ __launch_bounds__(256) void reduce_kernel(RdArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const T *__restrict__ X = static_cast<const T *>(a.x);
    const T *__restrict__ Wt = static_cast<const T *>(a.w);
    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    T *__restrict__ Y = static_cast<T *>(a.y);
    const int taps = a.KH * a.KW;
    const int terms = a.Cig * taps;
    for (int64_t e = wave0; e < a.count; e += nwaves) {
        int64_t r = e;
        const int ow = (int)(r % a.OW);
        r /= a.OW;
        const int oh = (int)(r % a.OH);
        r /= a.OH;
        const int co = (int)(r % a.C_out);
        const int64_t n = r / a.C_out;
        const int g = co / a.Cog;
        float acc = 0.f;
        for (int i = lane; i < terms; i += 64) {
            const int c = i / taps;
            const int t = i - c * taps;
            const int kh = t / a.KW, kw = t - kh * a.KW;
            const int ih = oh * a.SH - a.PH + kh * a.DH;
            const int iw = ow * a.SW - a.PW + kw * a.DW;
            if ((unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W) {
                const float xv = to_f32(X[n * a.xs_n + (int64_t)(g * a.Cig + c) * a.xs_c + (int64_t)ih * a.xs_h +
                                          (int64_t)iw * a.xs_w]);
                const float wv = to_f32(Wt[(int64_t)co * a.ws0 + (int64_t)c * a.ws1 + (int64_t)kh * a.ws2 +
                                           (int64_t)kw * a.ws3]);
                acc = __builtin_fmaf(xv, wv, acc);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (lane == 0) {
            if (a.has_bias) acc += to_f32(Bp[co]);
            Y[n * a.ys_n + (int64_t)co * a.ys_c + (int64_t)oh * a.ys_h + (int64_t)ow * a.ys_w] = from_f32<T>(acc);
        }
    }
}

void reduce_geometry(const conv_desc &d, conv_plan_t &p)
{
    const int64_t positions = d.out[0] * d.out[1];
    const int64_t count = d.N * d.C_out * positions;
    int64_t blocks = cdiv(count, 4);
    if (blocks > (1 << 20)) blocks = 1 << 20;
    p.grid[0] = blocks;
    p.block = 256;
    p.tile[0] = count;
    p.lds_bytes = 0;
}

int launch_reduce(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream)
{
    const conv_desc &d = p.d;
    RdArgs a;
    a.x = x;
    a.w = w;
    a.b = b;
    a.y = y;
    const bool two = d.spatial == 2;
    a.xs_n = d.x.strides[0];
    a.xs_c = d.x.strides[1];
    a.xs_h = two ? d.x.strides[2] : 0;
    a.xs_w = two ? d.x.strides[3] : d.x.strides[2];
    a.ys_n = p.y.strides[0];
    a.ys_c = p.y.strides[1];
    a.ys_h = two ? p.y.strides[2] : 0;
    a.ys_w = two ? p.y.strides[3] : p.y.strides[2];
    a.ws0 = d.w.strides[0];
    a.ws1 = d.w.strides[1];
    a.ws2 = two ? d.w.strides[2] : 0;
    a.ws3 = two ? d.w.strides[3] : d.w.strides[2];
    a.count = p.tile[0];
    a.G = (int32_t)d.groups;
    a.Cig = (int32_t)(d.C_in / d.groups);
    a.Cog = (int32_t)(d.C_out / d.groups);
    a.C_out = (int32_t)d.C_out;
    const int h = two ? 0 : -1, wd = two ? 1 : 0;
    auto at = [&](const int64_t *v, int i, int64_t dflt) { return (int32_t)(i < 0 ? dflt : v[i]); };
    a.H = at(d.in, h, 1);
    a.W = (int32_t)d.in[wd];
    a.OH = at(d.out, h, 1);
    a.OW = (int32_t)d.out[wd];
    a.KH = at(d.k, h, 1);
    a.KW = (int32_t)d.k[wd];
    a.SH = at(d.stride, h, 1);
    a.SW = (int32_t)d.stride[wd];
    a.PH = at(d.padding_before, h, 0);
    a.PW = (int32_t)d.padding_before[wd];
    a.DH = at(d.dilation, h, 1);
    a.DW = (int32_t)d.dilation[wd];
    a.has_bias = d.has_bias;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)p.grid[0]), block(256);
    switch (d.dtype) {
    case CONV_F32: hipLaunchKernelGGL(reduce_kernel<float>, grid, block, 0, s, a); break;
    case CONV_F16: hipLaunchKernelGGL(reduce_kernel<f16_t>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(reduce_kernel<bf16_t>, grid, block, 0, s, a); break;
    }
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
