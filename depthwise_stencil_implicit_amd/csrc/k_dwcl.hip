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
// the same pixel, so every wave load and store is one contiguous run.
// Workgroups are persistent -- one resident round over all CUs -- and each
// keeps one (strip chunk, channel chunk), so its weights are staged in LDS
// (fp32 [tap][channel]) once; each kernel row reads back only its K weights
// per channel.
//
// Loads are raw buffer loads: a lane's column offsets are computed once, the
// row offset (uniform across the wave) rides in the scalar offset, and absent
// rows or columns get an out-of-range offset so the hardware returns zeros --
// no branch for the padding.  The (output row, kernel row) steps form one
// rolled loop with a one-step prefetch, which keeps the register footprint
// near 120 VGPRs (four waves per SIMD) while a row segment is in flight.
// Accumulation is fp32 FMA, the bias is the initial value, and each result is
// rounded once to the output dtype.
#include "dev_common.h"
#include "internal.h"

#include <algorithm>

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

// Weight words per kernel row: 16-bit types keep K/2 packed column pairs
// (kw = 2p, 2p+1) and the last, odd column as fp32; fp32 keeps K fp32 taps.
template <typename T, int K> struct DwTaps {
    static constexpr bool DOT = Word<T>::V == 2;
    static constexpr int KP = DOT ? K / 2 : 0;
    static constexpr int WPR = DOT ? KP + 1 : K;
};

template <typename T, int K, int S, int TO>
__global__ __launch_bounds__(256) void dwcl_kernel(DwArgs a)
{
    constexpr int V = Word<T>::V;
    constexpr int ES = Dt<T>::size;
    constexpr int NCOL = (TO - 1) * S + K;
    constexpr int INVALID = 0x7fffff00;
    constexpr int M = (K + S - 1) / S;   // output rows open at once (accumulator slots)
    constexpr int U = M * S;             // input rows per unrolled block: slot pattern repeats
    constexpr bool DOT = DwTaps<T, K>::DOT;
    constexpr int KP = DwTaps<T, K>::KP;
    constexpr int WPR = DwTaps<T, K>::WPR;
    static_assert(!DOT || (K & 1), "pairs leave one odd column");
    extern __shared__ __attribute__((aligned(16))) uint32_t sw[];  // [K*WPR][CW + 2] words

    // Persistent workgroups: a workgroup keeps one (strip chunk, channel
    // chunk) for its whole life and walks one contiguous block of output rows
    // (n, oh).  Workgroup numbers are remapped so each XCD owns a contiguous
    // band of row blocks: neighbouring rows share K-1 input rows in its L2.
    const int tid = threadIdx.x;
    const int SC = a.strip_chunks * a.ch_chunks;
    const int vb = xcd_block(blockIdx.x, gridDim.x);
    const int sc = vb % SC;
    const int chc = sc % a.ch_chunks;
    const int stc = sc / a.ch_chunks;
    const int q = vb / SC;
    const int nwg = gridDim.x / SC;
    const int rows_total = a.N * a.OH;
    const int first = (int)((int64_t)q * rows_total / nwg);
    const int last = (int)((int64_t)(q + 1) * rows_total / nwg);

    // Stage this workgroup's weights once, entry (kh, j) of channel cl at
    // sw[(kh*WPR + j)*pitch + cl]: a packed pair of the stored 16-bit values
    // (j < KP) or one fp32 tap.
    const int CW = a.cpb * V;
    const int pitch = CW + 2;
    const int c_base = chc * CW;
    {
        const T *Wt = static_cast<const T *>(a.w);
        for (int i = tid; i < K * WPR * CW; i += 256) {
            const int cl = i / (K * WPR);
            const int e = i - cl * (K * WPR);
            const int kh = e / WPR, j = e - kh * WPR;
            const int c = min(c_base + cl, a.C - 1);
            const T *wr = Wt + (int64_t)c * a.ws0 + kh * a.ws2;
            uint32_t v;
            if constexpr (DOT) {
                if (j < KP) v = (uint32_t)wr[(2 * j) * a.ws3].u | ((uint32_t)wr[(2 * j + 1) * a.ws3].u << 16);
                else v = __float_as_uint(to_f32(wr[(K - 1) * a.ws3]));
            } else {
                v = __float_as_uint(to_f32(wr[j * a.ws3]));
            }
            sw[e * pitch + cl] = v;
        }
    }
    __syncthreads();

    const int cl0 = (tid % a.cpb) * V;
    const int c0 = c_base + cl0;
    const int strip = stc * a.spb + tid / a.cpb;
    if (c0 >= a.C || strip >= a.nstrips || tid >= a.cpb * a.spb || first >= last) return;
    const int ow0 = strip * TO;

    float bias[V];
    {
        const T *Bp = static_cast<const T *>(a.b);
#pragma unroll
        for (int v = 0; v < V; ++v) bias[v] = a.has_bias ? to_f32(Bp[c0 + v]) : 0.f;
    }

    // Column byte offsets of this lane's strip; absent columns are out of range.
    int vcol[NCOL];
    const int iw0 = ow0 * S - a.pb_w;
#pragma unroll
    for (int col = 0; col < NCOL; ++col) {
        const int iw = iw0 + col;
        vcol[col] = (unsigned)iw < (unsigned)a.W ? (iw * a.xs_w + c0) * ES : INVALID;
    }
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    T *__restrict__ Y = static_cast<T *>(a.y) + c0;
    const uint32_t *swl = sw + cl0;

    // The block of output rows splits into per-image segments.  In a segment
    // with output rows oh0 + j (j < nj), input row ih0 + i (ih0 = oh0*S - pb)
    // feeds output j at kernel row kh = i - j*S.  Input rows are streamed once;
    // output j lives in accumulator slot j mod M from its first input row to
    // its last (kh = K-1), where it is stored and its slot reset to the bias.
    // Unrolling the stream by U = M*S input rows makes every (slot, kh) pair a
    // compile-time constant.  Slots of rows outside the segment (j < 0 or
    // j >= nj) collect harmless partial sums that are never stored.
    for (int row0 = first; row0 < last;) {
        const int n = row0 / a.OH;
        const int oh0 = row0 - n * a.OH;
        const int nj = min(last - row0, a.OH - oh0);
        row0 += nj;
        const int ih0 = oh0 * S - a.pb_h;
        const int ni = (nj - 1) * S + K;   // input rows of the segment
        const int xbase = n * a.xs_n;
        T *Yn = Y + (int64_t)n * a.ys_n;

        float acc[M][TO][V];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int t = 0; t < TO; ++t)
#pragma unroll
                for (int v = 0; v < V; ++v) acc[m][t][v] = bias[v];

        auto fetch = [&](int i, uint32_t (&buf)[NCOL]) {
            const int ih = ih0 + i;
            const bool ok = (unsigned)ih < (unsigned)a.H && i < ni;
            const int soff = ok ? (xbase + ih * a.xs_h) * ES : 0;
            const int vbad = ok ? 0 : INVALID;
#pragma unroll
            for (int col = 0; col < NCOL; ++col)
                buf[col] = __builtin_amdgcn_raw_buffer_load_b32(xr, vcol[col] + vbad, soff, 0);
        };

        uint32_t cur[NCOL], nxt[NCOL];
        fetch(0, cur);
        for (int ib = 0; ib < ni; ib += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = ib + u;
                if (i < ni) {
                    fetch(i + 1, nxt);
                    // Row operands.  16-bit: the pair of columns (q, q+1) of each
                    // channel packed into one word, and the odd last column widened;
                    // fp32: every column as is.  Unused entries fold away.
                    uint32_t plo[NCOL], phi[NCOL];
                    float xv[NCOL][V];
#pragma unroll
                    for (int col = 0; col < NCOL; ++col) {
                        if constexpr (DOT) {
                            if (col + 1 < NCOL) {
                                plo[col] = (cur[col] & 0xffffu) | (cur[col + 1] << 16);
                                phi[col] = (cur[col] >> 16) | (cur[col + 1] & 0xffff0000u);
                            }
                        }
                        Word<T>::widen(cur[col], xv[col]);
                    }
                    // Open outputs j = J*M + jp with kh = u - jp*S in [0, K).
#pragma unroll
                    for (int jp = -M; jp <= M; ++jp) {
                        const int kh = u - jp * S;
                        if (kh < 0 || kh >= K) continue;
                        // Output j = ib/S + jp (ib is a multiple of U = M*S).  Rows
                        // outside the segment are skipped (a uniform branch), so the
                        // halo rows of a short segment cost loads but no arithmetic;
                        // a skipped slot still holds the bias when its next output
                        // (j + M, whose first input row follows j's last) opens it.
                        const int j = ib / S + jp;
                        if (j < 0 || j >= nj) continue;
                        const int slot = ((jp % M) + M) % M;
                        if constexpr (DOT) {
                            uint2 wp[KP];
#pragma unroll
                            for (int pp = 0; pp < KP; ++pp)
                                wp[pp] = *reinterpret_cast<const uint2 *>(swl + (kh * WPR + pp) * pitch);
                            const uint2 ws = *reinterpret_cast<const uint2 *>(swl + (kh * WPR + KP) * pitch);
#pragma unroll
                            for (int t = 0; t < TO; ++t) {
#pragma unroll
                                for (int pp = 0; pp < KP; ++pp) {
                                    acc[slot][t][0] = dot2<T>(plo[t * S + 2 * pp], wp[pp].x, acc[slot][t][0]);
                                    acc[slot][t][1] = dot2<T>(phi[t * S + 2 * pp], wp[pp].y, acc[slot][t][1]);
                                }
                                acc[slot][t][0] = __builtin_fmaf(xv[t * S + K - 1][0], __uint_as_float(ws.x), acc[slot][t][0]);
                                acc[slot][t][V - 1] =
                                    __builtin_fmaf(xv[t * S + K - 1][V - 1], __uint_as_float(ws.y), acc[slot][t][V - 1]);
                            }
                        } else {
                            float wk[K][V];
#pragma unroll
                            for (int kw = 0; kw < K; ++kw)
#pragma unroll
                                for (int v = 0; v < V; ++v) wk[kw][v] = __uint_as_float(swl[(kh * K + kw) * pitch + v]);
#pragma unroll
                            for (int t = 0; t < TO; ++t)
#pragma unroll
                                for (int kw = 0; kw < K; ++kw)
#pragma unroll
                                    for (int v = 0; v < V; ++v)
                                        acc[slot][t][v] = __builtin_fmaf(xv[t * S + kw][v], wk[kw][v], acc[slot][t][v]);
                        }
                        if (kh == K - 1) {
                            // Output j is complete.
                            T *yrow = Yn + (int64_t)(oh0 + j) * a.ys_h;
#pragma unroll
                            for (int t = 0; t < TO; ++t)
                                if (ow0 + t < a.OW)
                                    *reinterpret_cast<uint32_t *>(yrow + (int64_t)(ow0 + t) * a.ys_w) =
                                        Word<T>::narrow(acc[slot][t]);
#pragma unroll
                            for (int t = 0; t < TO; ++t)
#pragma unroll
                                for (int v = 0; v < V; ++v) acc[slot][t][v] = bias[v];
                        }
                    }
#pragma unroll
                    for (int col = 0; col < NCOL; ++col) cur[col] = nxt[col];
                }
            }
        }
    }
}

namespace {

template <typename T, int K, int S, int TO>
hipError_t go(DwArgs a, hipStream_t s)
{
    auto kern = dwcl_kernel<T, K, S, TO>;
    const size_t lds = (size_t)K * DwTaps<T, K>::WPR * (a.cpb * Word<T>::V + 2) * sizeof(uint32_t);
    // One resident round of persistent workgroups, a multiple of the number
    // of (strip, channel) chunks, and no more than there are rows to share.
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), 256, lds);
    if (e != hipSuccess) return e;
    const int64_t SC = (int64_t)a.strip_chunks * a.ch_chunks;
    int64_t slots = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
    const int64_t rows = (int64_t)a.N * a.OH;
    int64_t per_sc = std::max<int64_t>(1, std::min<int64_t>(slots / SC, rows));
    const int64_t grid = per_sc * SC;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const DwArgs &a, int k, int s, int to, hipStream_t st)
{
#define MICONV_DW(KK, SS, TT) \
    if (k == KK && s == SS && to == TT) return go<T, KK, SS, TT>(a, st);
    MICONV_DW(3, 1, 8) MICONV_DW(3, 1, 14) MICONV_DW(5, 1, 8) MICONV_DW(7, 1, 4) MICONV_DW(3, 2, 7)
    MICONV_DW(5, 2, 7) MICONV_DW(7, 2, 4)
#undef MICONV_DW
    return hipErrorInvalidValue;
}

}  // namespace

// Kernel sizes and strides with a compiled schedule (square kernels, equal strides).
bool dwcl_has_schedule(int64_t kh, int64_t kw, int64_t sh, int64_t sw)
{
    return kh == kw && sh == sw && (kh == 3 || kh == 5 || kh == 7) && (sh == 1 || sh == 2);
}

// Strip width (outputs per lane along W).  The rolling window holds
// ceil(K/S) * TO accumulators per channel, so wide kernels get narrow strips;
// among a kernel's compiled widths, the one wasting the fewest lanes on the
// last, partial strip of a row wins (ties: the first listed).
int dwcl_strip(int64_t k, int64_t s, int64_t ow)
{
    int cand[2] = {0, 0};
    if (s == 1) {
        if (k == 3) { cand[0] = 8; cand[1] = 14; }
        else if (k == 5) cand[0] = 8;
        else cand[0] = 4;
    } else {
        cand[0] = k == 7 ? 4 : 7;
    }
    int best = cand[0];
    int64_t waste = cdiv(ow, best) * best - ow;
    if (cand[1]) {
        const int64_t w2 = cdiv(ow, cand[1]) * cand[1] - ow;
        if (w2 < waste) best = cand[1];
    }
    return best;
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
