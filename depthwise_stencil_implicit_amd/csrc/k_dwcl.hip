// Depthwise 2-D stencil for channel-contiguous (channels-last) inputs
// (kernel CONV_K_DW_CL).
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: a direct
// stencil for depthwise convolutions with dilation 1 and kernels up to 9x9,
// with a register sliding-window schedule for channel-contiguous inputs.
//
// Layout on gfx950: x is [N][H][W][C] in memory (C fastest).  A lane owns one
// 32-bit word of channels (two 16-bit channels, or one fp32 channel) and a
// strip of TO consecutive output columns; it walks RPT output rows.  For each
// output row and kernel row it loads the (TO-1)*S + K input words of its strip
// left to right; each load is widened to fp32 once and feeds every output of
// the strip whose window covers that column -- the loaded row segment is the
// register sliding window.  Consecutive lanes hold consecutive channel words of
// the same pixel, so every wave load and store is one contiguous run.  All
// K*K weights of the lane's channels live in registers as fp32 for the whole
// kernel: no LDS and no barrier.
//
// Loads are raw buffer loads whose out-of-range offsets return zero, so the
// zero padding costs no branch and all loads of a row can be in flight at once.
// Accumulation is fp32 FMA, the bias is the initial value, and each result is
// rounded once to the output dtype.
#include "dev_common.h"
#include "internal.h"

namespace miconv {

struct DwArgs {
    const void *x, *w, *b;
    void *y;
    int64_t ys_n, ys_h, ys_w;         // element strides of y (channel stride 1)
    int32_t xs_n, xs_h, xs_w;         // element strides of x (channel stride 1), 32-bit
    int32_t x_bytes;                  // bytes addressable from x (buffer range)
    int64_t ws0, ws2, ws3;            // weight strides (output channel, kh, kw)
    int32_t N, H, W, C, OH, OW, pb_h, pb_w;
    int32_t cpb, spb, rpt;            // lane words / strips per workgroup, rows per thread
    int32_t ch_chunks, strip_chunks, row_chunks, nstrips, total;
    int32_t has_bias;
};

__device__ __forceinline__ int xcd_block(int b, int total)
{
    const int q = total >> 3, r = total & 7;
    const int xcd = b & 7, local = b >> 3;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

template <typename T> struct Word;
template <> struct Word<bf16_t> {
    static constexpr int V = 2;
    __device__ static void widen(uint32_t u, float (&f)[2]) { f[0] = lo_f32(u, bf16_t{}); f[1] = hi_f32(u, bf16_t{}); }
    __device__ static uint32_t narrow(const float (&f)[2]) { return pack2<bf16_t>(f[0], f[1]); }
};
template <> struct Word<f16_t> {
    static constexpr int V = 2;
    __device__ static void widen(uint32_t u, float (&f)[2]) { f[0] = lo_f32(u, f16_t{}); f[1] = hi_f32(u, f16_t{}); }
    __device__ static uint32_t narrow(const float (&f)[2]) { return pack2<f16_t>(f[0], f[1]); }
};
template <> struct Word<float> {
    static constexpr int V = 1;
    __device__ static void widen(uint32_t u, float (&f)[1]) { f[0] = __uint_as_float(u); }
    __device__ static uint32_t narrow(const float (&f)[1]) { return __float_as_uint(f[0]); }
};

template <typename T, int K, int S, int TO>
__global__ __launch_bounds__(256) void dwcl_kernel(DwArgs a)
{
    constexpr int V = Word<T>::V;
    constexpr int ES = Dt<T>::size;
    constexpr int NCOL = (TO - 1) * S + K;

    const int tid = threadIdx.x;
    int blk = xcd_block(blockIdx.x, a.total);
    const int chc = blk % a.ch_chunks;
    blk /= a.ch_chunks;
    const int stc = blk % a.strip_chunks;
    blk /= a.strip_chunks;
    const int rowc = blk % a.row_chunks;
    const int n = blk / a.row_chunks;

    const int word = chc * a.cpb + tid % a.cpb;     // channel word index
    const int c0 = word * V;
    const int strip = stc * a.spb + tid / a.cpb;
    if (c0 >= a.C || strip >= a.nstrips) return;
    const int ow0 = strip * TO;

    // Weights of this lane's channels, fp32, in registers.
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.w), (short)0,
                                                                        0x7fffffff, 0x00020000);
    const T *Wt = static_cast<const T *>(a.w);
    float wv[K][K][V];
#pragma unroll
    for (int kh = 0; kh < K; ++kh)
#pragma unroll
        for (int kw = 0; kw < K; ++kw)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int c = min(c0 + v, a.C - 1);
                wv[kh][kw][v] = to_f32(Wt[(int64_t)c * a.ws0 + kh * a.ws2 + kw * a.ws3]);
            }
    (void)wr;
    float bias[V];
    {
        const T *Bp = static_cast<const T *>(a.b);
#pragma unroll
        for (int v = 0; v < V; ++v) bias[v] = a.has_bias ? to_f32(Bp[min(c0 + v, a.C - 1)]) : 0.f;
    }

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    const int xbase = n * a.xs_n + c0;              // element offset of (n, 0, 0, c0)
    const int iw0 = ow0 * S - a.pb_w;
    T *__restrict__ Y = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + c0;

    const int oh_beg = rowc * a.rpt;
    const int oh_end = min(a.OH, oh_beg + a.rpt);
    for (int oh = oh_beg; oh < oh_end; ++oh) {
        float acc[TO][V];
#pragma unroll
        for (int t = 0; t < TO; ++t)
#pragma unroll
            for (int v = 0; v < V; ++v) acc[t][v] = bias[v];
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            const int ih = oh * S - a.pb_h + kh;
            const bool row_ok = (unsigned)ih < (unsigned)a.H;
            const int rbase = xbase + ih * a.xs_h;
#pragma unroll
            for (int col = 0; col < NCOL; ++col) {
                const int iw = iw0 + col;
                const bool ok = row_ok && (unsigned)iw < (unsigned)a.W;
                const int off = ok ? (rbase + iw * a.xs_w) * ES : 0x7fffffff;
                const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
                float xv[V];
                Word<T>::widen(u, xv);
#pragma unroll
                for (int t = 0; t < TO; ++t) {
                    const int kw = col - t * S;
                    if (kw >= 0 && kw < K) {
#pragma unroll
                        for (int v = 0; v < V; ++v) acc[t][v] = __builtin_fmaf(xv[v], wv[kh][kw][v], acc[t][v]);
                    }
                }
            }
        }
        T *yrow = Y + (int64_t)oh * a.ys_h;
#pragma unroll
        for (int t = 0; t < TO; ++t) {
            if (ow0 + t < a.OW) {
                const uint32_t u = Word<T>::narrow(acc[t]);
                *reinterpret_cast<uint32_t *>(yrow + (int64_t)(ow0 + t) * a.ys_w) = u;
            }
        }
    }
}

namespace {

template <typename T, int K, int S, int TO>
hipError_t go(const DwArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((dwcl_kernel<T, K, S, TO>), dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const DwArgs &a, int k, int s, int to, hipStream_t st)
{
#define MICONV_DW(KK, SS, TT) \
    if (k == KK && s == SS && to == TT) return go<T, KK, SS, TT>(a, st);
    MICONV_DW(3, 1, 14) MICONV_DW(3, 1, 8) MICONV_DW(5, 1, 14) MICONV_DW(5, 1, 8) MICONV_DW(7, 1, 14)
    MICONV_DW(7, 1, 8) MICONV_DW(3, 2, 7) MICONV_DW(3, 2, 4) MICONV_DW(5, 2, 7) MICONV_DW(5, 2, 4)
    MICONV_DW(7, 2, 7) MICONV_DW(7, 2, 4)
#undef MICONV_DW
    return hipErrorInvalidValue;
}

}  // namespace

// Kernel sizes and strides with a compiled schedule (square kernels, equal strides).
bool dwcl_has_schedule(int64_t kh, int64_t kw, int64_t sh, int64_t sw)
{
    return kh == kw && sh == sw && (kh == 3 || kh == 5 || kh == 7) && (sh == 1 || sh == 2);
}

// Strip width (outputs per lane along W): the candidate that wastes the fewest
// lanes on the last, partial strip of a row.
int dwcl_strip(int64_t s, int64_t ow)
{
    const int a = s == 1 ? 14 : 7, b = s == 1 ? 8 : 4;
    const int64_t wa = cdiv(ow, a) * a - ow, wb = cdiv(ow, b) * b - ow;
    return wa <= wb ? a : b;
}

int launch_dwcl(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream, bool vec)
{
    (void)vec;
    const conv_desc &d = p.d;
    DwArgs a;
    a.x = x;
    a.w = w;
    a.b = b;
    a.y = y;
    a.xs_n = (int32_t)d.x.strides[0];
    a.xs_h = (int32_t)d.x.strides[2];
    a.xs_w = (int32_t)d.x.strides[3];
    a.x_bytes = (int32_t)p.tile[7];
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
    a.cpb = (int32_t)p.tile[1];
    a.spb = (int32_t)p.tile[2];
    a.rpt = (int32_t)p.tile[3];
    a.ch_chunks = (int32_t)p.tile[4];
    a.strip_chunks = (int32_t)p.tile[5];
    a.row_chunks = (int32_t)p.tile[6];
    a.nstrips = (int32_t)cdiv(d.out[1], p.tile[0]);
    a.total = (int32_t)p.grid[0];
    a.has_bias = d.has_bias;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const int k = (int)d.k[0], st = (int)d.stride[0], to = (int)p.tile[0];
    switch (d.dtype) {
    case CONV_F32: e = dispatch<float>(a, k, st, to, s); break;
    case CONV_F16: e = dispatch<f16_t>(a, k, st, to, s); break;
    default: e = dispatch<bf16_t>(a, k, st, to, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
