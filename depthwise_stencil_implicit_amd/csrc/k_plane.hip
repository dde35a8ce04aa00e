// Depthwise / few-channel grouped 2-D stencil for any memory layout
// (kernel CONV_K_PLANE).
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: the direct
// stencil covers depthwise convolutions and grouped ones with up to 8 input
// channels per group and any channel multiplier, NCHW or channels-last
// inputs, an optional bias and asymmetric padding; its portable base schedule
// is the one every layout can use, and a multiplier schedule computes all
// output channels of an input channel from one load.
//
// Layout on gfx950: one workgroup owns one (image, group) pair and a TH x TW
// tile of output positions.  It first copies the input halo tile of the
// group's Cig channels -- (TH-1)*SH + (KH-1)*DH + 1 rows by the same in
// columns -- into LDS as fp32, zero where the window leaves the input, so the
// tap loop has no bounds checks.  Each thread then owns R vertically adjacent
// outputs of one column and walks the output channels of the group MB at a
// time: the MB x R accumulators stay in registers, so every LDS read of an
// input value feeds MB output channels (the multiplier fan-out).  Weights are
// read with workgroup-uniform addresses.  Rows of NCHW inputs are loaded by
// consecutive threads, so the staging loads are coalesced for NCHW; other
// layouts are correct but strided.  fp32 accumulation, bias added before the
// single rounding.
#include "dev_common.h"
#include "internal.h"

namespace miconv {

struct PlArgs {
    const void *x, *w, *b;
    void *y;
    int64_t xs_n, xs_c, xs_h, xs_w;
    int64_t ys_n, ys_c, ys_h, ys_w;
    int64_t ws0, ws1, ws2, ws3;
    int32_t N, G, Cig, Cog, H, W, OH, OW, KH, KW, SH, SW, PH, PW, DH, DW;
    int32_t TH, TW, R, IH, IW, tiles_h, tiles_w, total, has_bias;
};

template <typename T, int MB, int R>
__global__ __launch_bounds__(256) void plane_kernel(PlArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float sx[];  // [Cig][IH][IW]
    const int tid = threadIdx.x;
    int blk = blockIdx.x;
    const int tw = blk % a.tiles_w;
    blk /= a.tiles_w;
    const int th = blk % a.tiles_h;
    blk /= a.tiles_h;
    const int g = blk % a.G;
    const int n = blk / a.G;

    const T *__restrict__ X = static_cast<const T *>(a.x) + (int64_t)n * a.xs_n + (int64_t)g * a.Cig * a.xs_c;
    const int ih0 = th * a.TH * a.SH - a.PH;
    const int iw0 = tw * a.TW * a.SW - a.PW;
    const int plane = a.IH * a.IW;
    const int halo = a.Cig * plane;
    // SL values per thread per pass, all loads issued before the first LDS
    // write, so their latencies overlap.
    constexpr int SL = 4;
    for (int i0 = tid; i0 < halo; i0 += SL * 256) {
        float v[SL];
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int i = i0 + u * 256;
            const int c = i / plane;
            const int rem = i - c * plane;
            const int r = rem / a.IW, q = rem - r * a.IW;
            const int ih = ih0 + r, iw = iw0 + q;
            v[u] = 0.f;
            if (i < halo && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W)
                v[u] = to_f32(X[(int64_t)c * a.xs_c + (int64_t)ih * a.xs_h + (int64_t)iw * a.xs_w]);
        }
#pragma unroll
        for (int u = 0; u < SL; ++u)
            if (i0 + u * 256 < halo) sx[i0 + u * 256] = v[u];
    }
    __syncthreads();

    const int tx = tid % a.TW;
    const int ty = tid / a.TW;
    const int ow = tw * a.TW + tx;
    const int ohb = th * a.TH + ty * R;
    if (ty * R >= a.TH || ow >= a.OW || ohb >= a.OH) return;

    const T *__restrict__ Wt = static_cast<const T *>(a.w);
    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    T *__restrict__ Y = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + (int64_t)ow * a.ys_w;
    const int lrow = ty * R * a.SH;
    const int lcol = tx * a.SW;

    for (int j0 = 0; j0 < a.Cog; j0 += MB) {
        float acc[MB][R];
#pragma unroll
        for (int jj = 0; jj < MB; ++jj) {
            const int co = g * a.Cog + j0 + jj;
            const float bv = (a.has_bias && j0 + jj < a.Cog) ? to_f32(Bp[co]) : 0.f;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) acc[jj][rr] = bv;
        }
        for (int c = 0; c < a.Cig; ++c) {
            const float *sp = sx + c * plane;
            for (int kh = 0; kh < a.KH; ++kh) {
                for (int kw = 0; kw < a.KW; ++kw) {
                    float xv[R];
#pragma unroll
                    for (int rr = 0; rr < R; ++rr)
                        xv[rr] = sp[(lrow + rr * a.SH + kh * a.DH) * a.IW + lcol + kw * a.DW];
#pragma unroll
                    for (int jj = 0; jj < MB; ++jj) {
                        const int j = min(j0 + jj, a.Cog - 1);
                        const float wv = to_f32(Wt[(int64_t)(g * a.Cog + j) * a.ws0 + (int64_t)c * a.ws1 +
                                                   (int64_t)kh * a.ws2 + (int64_t)kw * a.ws3]);
#pragma unroll
                        for (int rr = 0; rr < R; ++rr) acc[jj][rr] = __builtin_fmaf(xv[rr], wv, acc[jj][rr]);
                    }
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < MB; ++jj) {
            if (j0 + jj >= a.Cog) break;
            const int64_t co = g * a.Cog + j0 + jj;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const int oh = ohb + rr;
                if (oh < a.OH) Y[co * a.ys_c + (int64_t)oh * a.ys_h] = from_f32<T>(acc[jj][rr]);
            }
        }
    }
}

namespace {

template <typename T, int MB>
hipError_t go(const PlArgs &a, int R, size_t lds, hipStream_t s)
{
    if (R == 1)
        hipLaunchKernelGGL((plane_kernel<T, MB, 1>), dim3(a.total), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL((plane_kernel<T, MB, 2>), dim3(a.total), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const PlArgs &a, int mb, size_t lds, hipStream_t s)
{
    switch (mb) {
    case 1: return go<T, 1>(a, a.R, lds, s);
    case 2: return go<T, 2>(a, a.R, lds, s);
    case 4: return go<T, 4>(a, a.R, lds, s);
    case 8: return go<T, 8>(a, a.R, lds, s);
    default: return go<T, 16>(a, a.R, lds, s);
    }
}

}  // namespace

int launch_plane(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream)
{
    const conv_desc &d = p.d;
    PlArgs a;
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
    const int h = two ? 0 : -1, wd = two ? 1 : 0;
    auto at = [&](const int64_t *v, int i, int64_t dflt) { return i < 0 ? dflt : v[i]; };
    a.N = (int32_t)d.N;
    a.G = (int32_t)d.groups;
    a.Cig = (int32_t)(d.C_in / d.groups);
    a.Cog = (int32_t)(d.C_out / d.groups);
    a.H = (int32_t)at(d.in, h, 1);
    a.W = (int32_t)d.in[wd];
    a.OH = (int32_t)at(d.out, h, 1);
    a.OW = (int32_t)d.out[wd];
    a.KH = (int32_t)at(d.k, h, 1);
    a.KW = (int32_t)d.k[wd];
    a.SH = (int32_t)at(d.stride, h, 1);
    a.SW = (int32_t)d.stride[wd];
    a.PH = (int32_t)at(d.padding_before, h, 0);
    a.PW = (int32_t)d.padding_before[wd];
    a.DH = (int32_t)at(d.dilation, h, 1);
    a.DW = (int32_t)d.dilation[wd];
    a.TH = (int32_t)p.tile[0];
    a.TW = (int32_t)p.tile[1];
    a.R = (int32_t)p.tile[2];
    a.IH = (int32_t)p.tile[4];
    a.IW = (int32_t)p.tile[5];
    a.tiles_h = (int32_t)p.tile[6];
    a.tiles_w = (int32_t)p.tile[7];
    a.total = (int32_t)p.grid[0];
    a.has_bias = d.has_bias;
    const int mb = (int)p.tile[3];
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (d.dtype) {
    case CONV_F32: e = dispatch<float>(a, mb, (size_t)p.lds_bytes, s); break;
    case CONV_F16: e = dispatch<f16_t>(a, mb, (size_t)p.lds_bytes, s); break;
    default: e = dispatch<bf16_t>(a, mb, (size_t)p.lds_bytes, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
