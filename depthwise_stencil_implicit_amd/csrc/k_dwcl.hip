// Depthwise 2-D stencil for channel-contiguous (channels-last) inputs
// (kernel CONV_K_DW_CL).
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: a direct
// stencil for depthwise convolutions with dilation 1 and kernels up to 9x9,
// with a register sliding window schedule for channel-contiguous inputs.
//
// Layout on gfx950: x is [N][H][W][C] in memory (C fastest).  A lane owns one
// 16-byte vector of V consecutive channels and a strip of TO consecutive output
// columns of one output row at a time.  For each kernel row it walks the
// (TO-1)*S + KW input columns of the strip once, left to right: each 16-byte
// load (V channels of one pixel) is widened to fp32 once and feeds every output
// of the strip whose window covers that column, so the loaded row segment is
// the register sliding window.  Lanes of a wave hold consecutive channel
// vectors of the same pixels, so every load and store of the wave is one
// contiguous run of C elements.  Weights of the workgroup's channels are staged
// once in LDS as fp32 [KH][KW][channels].  Accumulation is fp32 FMA; the bias
// is added first and the result rounded once to the output dtype.
#include "dev_common.h"
#include "internal.h"

namespace miconv {

struct DwArgs {
    const void *x, *w, *b;
    void *y;
    int64_t xs_n, xs_h, xs_w;  // channel stride is 1
    int64_t ys_n, ys_h, ys_w;  // channel stride is 1
    int64_t ws0, ws2, ws3;     // weight strides (output channel, kh, kw)
    int32_t N, H, W, C, OH, OW, pb_h, pb_w;
    int32_t cvb, sp, rh;       // channel vectors / strips / rows per workgroup
    int32_t ch_chunks, col_chunks, row_chunks, total;
    int32_t has_bias;
};

template <typename T, int V, bool VEC>
__device__ __forceinline__ void load_vec(const T *p, int c, int C, bool inb, float (&out)[V])
{
    if (VEC) {
        if (inb) {
            if constexpr (Dt<T>::size == 2) {
                const uint4 u = *reinterpret_cast<const uint4 *>(p);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    out[2 * i] = lo_f32(w4[i], T{});
                    out[2 * i + 1] = hi_f32(w4[i], T{});
                }
            } else {
                const float4 f = *reinterpret_cast<const float4 *>(p);
                out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v) out[v] = 0.f;
        }
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) out[v] = (inb && c + v < C) ? to_f32(p[v]) : 0.f;
    }
}

template <typename T, int V, bool VEC>
__device__ __forceinline__ void store_vec(T *p, int c, int C, const float (&v)[V])
{
    if (VEC) {
        if constexpr (Dt<T>::size == 2) {
            uint4 u;
            u.x = pack2<T>(v[0], v[1]);
            u.y = pack2<T>(v[2], v[3]);
            u.z = pack2<T>(v[4], v[5]);
            u.w = pack2<T>(v[6], v[7]);
            *reinterpret_cast<uint4 *>(p) = u;
        } else {
            *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
            if (c + i < C) p[i] = from_f32<T>(v[i]);
    }
}

__device__ __forceinline__ int xcd_block(int b, int total)
{
    const int q = total >> 3, r = total & 7;
    const int xcd = b & 7, local = b >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

template <typename T, int KH, int KW, int S, int TO, bool VEC>
__global__ __launch_bounds__(256) void dwcl_kernel(DwArgs a)
{
    constexpr int V = 16 / Dt<T>::size;
    constexpr int NCOL = (TO - 1) * S + KW;
    extern __shared__ __attribute__((aligned(16))) float sw[];  // [KH][KW][cvb*V]

    const int tid = threadIdx.x;
    int blk = xcd_block(blockIdx.x, a.total);
    const int chc = blk % a.ch_chunks;
    blk /= a.ch_chunks;
    const int colc = blk % a.col_chunks;
    blk /= a.col_chunks;
    const int rowc = blk % a.row_chunks;
    const int n = blk / a.row_chunks;

    const int CW = a.cvb * V;  // channels per workgroup
    const int c_base = chc * CW;
    const T *__restrict__ Wt = static_cast<const T *>(a.w);
    for (int i = tid; i < KH * KW * CW; i += blockDim.x) {
        const int cl = i % CW;
        const int kk = i / CW;
        const int kw = kk % KW, kh = kk / KW;
        const int c = c_base + cl;
        sw[i] = c < a.C ? to_f32(Wt[c * a.ws0 + kh * a.ws2 + kw * a.ws3]) : 0.f;
    }
    __syncthreads();

    const int cvl = tid % a.cvb;
    const int sp = tid / a.cvb;
    if (sp >= a.sp) return;
    const int c0 = c_base + cvl * V;
    if (c0 >= a.C) return;
    const int ow0 = (colc * a.sp + sp) * TO;
    if (ow0 >= a.OW) return;

    float bias[V];
    {
        const T *Bp = static_cast<const T *>(a.b);
#pragma unroll
        for (int v = 0; v < V; ++v) bias[v] = (a.has_bias && c0 + v < a.C) ? to_f32(Bp[c0 + v]) : 0.f;
    }

    const T *__restrict__ X = static_cast<const T *>(a.x) + (int64_t)n * a.xs_n + c0;
    T *__restrict__ Y = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + c0;
    const int iw0 = ow0 * S - a.pb_w;
    const float *swl = sw + cvl * V;

    const int oh_end = min(a.OH, (rowc + 1) * a.rh);
    for (int oh = rowc * a.rh; oh < oh_end; ++oh) {
        float acc[TO][V];
#pragma unroll
        for (int t = 0; t < TO; ++t)
#pragma unroll
            for (int v = 0; v < V; ++v) acc[t][v] = bias[v];

#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
            const int ih = oh * S - a.pb_h + kh;
            if ((unsigned)ih >= (unsigned)a.H) continue;
            float wv[KW][V];
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) {
                const float *q = swl + (kh * KW + kw) * CW;
#pragma unroll
                for (int v = 0; v < V; v += 4) {
                    const float4 f = *reinterpret_cast<const float4 *>(q + v);
                    wv[kw][v] = f.x; wv[kw][v + 1] = f.y; wv[kw][v + 2] = f.z; wv[kw][v + 3] = f.w;
                }
            }
            const T *row = X + (int64_t)ih * a.xs_h;
#pragma unroll
            for (int col = 0; col < NCOL; ++col) {
                const int iw = iw0 + col;
                float xv[V];
                load_vec<T, V, VEC>(row + (int64_t)iw * a.xs_w, c0, a.C, (unsigned)iw < (unsigned)a.W, xv);
#pragma unroll
                for (int t = 0; t < TO; ++t) {
                    const int kw = col - t * S;
                    if (kw >= 0 && kw < KW) {
#pragma unroll
                        for (int v = 0; v < V; ++v) acc[t][v] = __builtin_fmaf(xv[v], wv[kw][v], acc[t][v]);
                    }
                }
            }
        }
        T *yrow = Y + (int64_t)oh * a.ys_h;
#pragma unroll
        for (int t = 0; t < TO; ++t)
            if (ow0 + t < a.OW) store_vec<T, V, VEC>(yrow + (int64_t)(ow0 + t) * a.ys_w, c0, a.C, acc[t]);
    }
}

namespace {

template <typename T, int KH, int KW, int S, int TO>
hipError_t go(const DwArgs &a, bool vec, size_t lds, hipStream_t s)
{
    if (vec)
        hipLaunchKernelGGL((dwcl_kernel<T, KH, KW, S, TO, true>), dim3(a.total), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL((dwcl_kernel<T, KH, KW, S, TO, false>), dim3(a.total), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const DwArgs &a, int k, int s, bool vec, size_t lds, hipStream_t st)
{
    // Strip width: 8 output columns at stride 1, 4 at stride 2.
    if (s == 1) {
        if (k == 3) return go<T, 3, 3, 1, 8>(a, vec, lds, st);
        if (k == 5) return go<T, 5, 5, 1, 8>(a, vec, lds, st);
        if (k == 7) return go<T, 7, 7, 1, 8>(a, vec, lds, st);
    } else if (s == 2) {
        if (k == 3) return go<T, 3, 3, 2, 4>(a, vec, lds, st);
        if (k == 5) return go<T, 5, 5, 2, 4>(a, vec, lds, st);
        if (k == 7) return go<T, 7, 7, 2, 4>(a, vec, lds, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Kernel sizes and strides with a compiled schedule (square kernels, equal strides).
bool dwcl_has_schedule(int64_t kh, int64_t kw, int64_t sh, int64_t sw)
{
    return kh == kw && sh == sw && (kh == 3 || kh == 5 || kh == 7) && (sh == 1 || sh == 2);
}

int dwcl_strip(int64_t s) { return s == 1 ? 8 : 4; }

int launch_dwcl(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream, bool vec)
{
    const conv_desc &d = p.d;
    DwArgs a;
    a.x = x;
    a.w = w;
    a.b = b;
    a.y = y;
    a.xs_n = d.x.strides[0];
    a.xs_h = d.x.strides[2];
    a.xs_w = d.x.strides[3];
    a.ys_n = p.y.strides[0];
    a.ys_h = p.y.strides[2];
    a.ys_w = p.y.strides[3];
    a.ws0 = d.w.strides[0];
    a.ws2 = d.w.strides[2];
    a.ws3 = d.w.strides[3];
    a.N = (int32_t)d.N;
    a.H = (int32_t)d.in[0];
    a.W = (int32_t)d.in[1];
    a.C = (int32_t)d.C_in;
    a.OH = (int32_t)d.out[0];
    a.OW = (int32_t)d.out[1];
    a.pb_h = (int32_t)d.padding_before[0];
    a.pb_w = (int32_t)d.padding_before[1];
    a.cvb = (int32_t)p.tile[1];
    a.sp = (int32_t)p.tile[2];
    a.rh = (int32_t)p.tile[3];
    a.ch_chunks = (int32_t)p.tile[4];
    a.col_chunks = (int32_t)p.tile[5];
    a.row_chunks = (int32_t)p.tile[6];
    a.total = (int32_t)p.grid[0];
    a.has_bias = d.has_bias;
    const size_t lds = (size_t)p.lds_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const int k = (int)d.k[0], st = (int)d.stride[0];
    switch (d.dtype) {
    case CONV_F32: e = dispatch<float>(a, k, st, vec, lds, s); break;
    case CONV_F16: e = dispatch<f16_t>(a, k, st, vec, lds, s); break;
    default: e = dispatch<bf16_t>(a, k, st, vec, lds, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
