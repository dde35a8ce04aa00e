// Few-channel grouped 2-D stencil with packed dot2 (kernel CONV_K_GRP).
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: grouped
// convolutions with up to 8 input channels per group and any channel
// multiplier, served by a schedule that computes a group's output channels
// from shared, once-loaded weights.
//
// Layout on gfx950 (fp16 / bf16 only): one workgroup owns one (image, group)
// pair and a tile of TH output rows by TW output columns.  The group's Cig
// input channels are staged once in LDS as packed channel pairs -- one 32-bit
// word holds input channels (2p, 2p+1) at one position -- zero-filled where
// the window leaves the input and for the missing partner of an odd channel
// count, so the padding and the odd channel contribute exact zeros.  The
// weights are staged as the matching pairs, [pair][tap][output channel].
// A thread owns P output positions of one row, interleaved with its
// neighbours' (thread tx of a row takes columns tx, tx + tpr, ...: consecutive
// lanes read consecutive LDS words and store consecutive elements), and JB
// output channels in registers: for every (pair, tap) it reads P input words
// and JB weight words (uniform addresses: LDS broadcast) and issues P*JB
// v_dot2_f32_{f16,bf16}, each doing both channels of the pair with fp32
// accumulation -- half the VALU instructions of one FMA per product, with no
// widening.  Any input strides (row-contiguous NCHW loads coalesce); the
// output tile is stored at y's strides, the bias added before one rounding.
#include "dev_common.h"
#include "internal.h"

#include <algorithm>

namespace miconv {

struct GpArgs {
    const void *x, *w, *b;
    void *y;
    int64_t xs_n, xs_c, xs_h, xs_w;
    int64_t ys_n, ys_c, ys_h, ys_w;
    int64_t ws0, ws1, ws2, ws3;
    int32_t N, G, Cig, Cog, H, W, OH, OW, KH, KW, SH, SW, PH, PW, DH, DW;
    int32_t TH, TW, IH, IW, tpr, tiles_h, tiles_w, total, has_bias, npairs, cog_pad;
};

template <typename T, int P, int JB>
__global__ __launch_bounds__(256) void grp_kernel(GpArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    const int taps = a.KH * a.KW;
    uint32_t *sw = smem;                                    // [npairs][taps][cog_pad]
    uint32_t *sx = smem + a.npairs * taps * a.cog_pad;      // [npairs][IH][IW]

    const int tid = threadIdx.x;
    int blk = blockIdx.x;
    const int tw = blk % a.tiles_w;
    blk /= a.tiles_w;
    const int th = blk % a.tiles_h;
    blk /= a.tiles_h;
    const int g = blk % a.G;
    const int n = blk / a.G;

    const T *__restrict__ X = static_cast<const T *>(a.x);
    const T *__restrict__ Wt = static_cast<const T *>(a.w);

    // Weights as channel pairs; pad channels (odd Cig, j >= Cog) are zero.
    for (int i = tid; i < a.npairs * taps * a.cog_pad; i += blockDim.x) {
        const int j = i % a.cog_pad;
        const int rest = i / a.cog_pad;
        const int tap = rest % taps;
        const int p = rest / taps;
        const int kh = tap / a.KW, kw = tap - kh * a.KW;
        uint32_t word = 0;
        if (j < a.Cog) {
            const int64_t base = (int64_t)(g * a.Cog + j) * a.ws0 + (int64_t)kh * a.ws2 + (int64_t)kw * a.ws3;
            const uint16_t lo = Wt[base + (int64_t)(2 * p) * a.ws1].u;
            const uint16_t hi = (2 * p + 1 < a.Cig) ? Wt[base + (int64_t)(2 * p + 1) * a.ws1].u : (uint16_t)0;
            word = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        sw[i] = word;
    }
    // Input halo tile as channel pairs; out-of-range and pad channels are zero.
    const int ih0 = th * a.TH * a.SH - a.PH;
    const int iw0 = tw * a.TW * a.SW - a.PW;
    const int plane = a.IH * a.IW;
    const T *Xg = X + (int64_t)n * a.xs_n + (int64_t)g * a.Cig * a.xs_c;
    for (int i = tid; i < a.npairs * plane; i += blockDim.x) {
        const int p = i / plane;
        const int rem = i - p * plane;
        const int r = rem / a.IW, q = rem - r * a.IW;
        const int ih = ih0 + r, iw = iw0 + q;
        uint32_t word = 0;
        if ((unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W) {
            const int64_t pos = (int64_t)ih * a.xs_h + (int64_t)iw * a.xs_w;
            const uint16_t lo = Xg[pos + (int64_t)(2 * p) * a.xs_c].u;
            const uint16_t hi = (2 * p + 1 < a.Cig) ? Xg[pos + (int64_t)(2 * p + 1) * a.xs_c].u : (uint16_t)0;
            word = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        sx[i] = word;
    }
    __syncthreads();

    const int ty = tid / a.tpr;
    const int tx = tid - ty * a.tpr;
    const int oh = th * a.TH + ty;
    const int ow0 = tw * a.TW + tx;
    if (ty >= a.TH || oh >= a.OH || ow0 >= a.OW) return;

    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    T *__restrict__ Y = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + (int64_t)oh * a.ys_h;
    const int lrow = ty * a.SH;
    const int lcol = tx * a.SW;

    for (int j0 = 0; j0 < a.Cog; j0 += JB) {
        float acc[P][JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const float bv = (a.has_bias && j0 + jj < a.Cog) ? to_f32(Bp[g * a.Cog + j0 + jj]) : 0.f;
#pragma unroll
            for (int p = 0; p < P; ++p) acc[p][jj] = bv;
        }
        for (int pr = 0; pr < a.npairs; ++pr) {
            const uint32_t *sxp = sx + pr * plane;
            for (int kh = 0; kh < a.KH; ++kh) {
                const uint32_t *srow = sxp + (lrow + kh * a.DH) * a.IW + lcol;
                for (int kw = 0; kw < a.KW; ++kw) {
                    uint32_t xv[P];
#pragma unroll
                    for (int p = 0; p < P; ++p) xv[p] = srow[p * a.tpr * a.SW + kw * a.DW];
                    const uint32_t *wrow = sw + (pr * taps + kh * a.KW + kw) * a.cog_pad + j0;
                    uint32_t wv[JB];
#pragma unroll
                    for (int jj = 0; jj < JB; jj += 4) {
                        const uint4 q = *reinterpret_cast<const uint4 *>(wrow + jj);
                        wv[jj] = q.x;
                        wv[jj + 1] = q.y;
                        wv[jj + 2] = q.z;
                        wv[jj + 3] = q.w;
                    }
#pragma unroll
                    for (int p = 0; p < P; ++p)
#pragma unroll
                        for (int jj = 0; jj < JB; ++jj) acc[p][jj] = dot2<T>(xv[p], wv[jj], acc[p][jj]);
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            if (j0 + jj >= a.Cog) break;
            T *yc = Y + (int64_t)(g * a.Cog + j0 + jj) * a.ys_c;
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (ow0 + p * a.tpr < a.OW) yc[(int64_t)(ow0 + p * a.tpr) * a.ys_w] = from_f32<T>(acc[p][jj]);
        }
    }
}

// Persistent schedule for kernels with a compile-time extent (KH x KW, KH in
// {1, KW}, KW in {3, 5, 7}), dilation 1, 32-bit element offsets and a tile
// of at most 8 words of channel pairs per thread.  Workgroup w serves group
// w mod G for every tile (image, tile row, tile column) j = w / G,
// w / G + wpg, ...: the group's weights are staged once, and while the tile
// in LDS is multiplied, the next tile's inputs are already in flight into
// registers (two 16-bit loads per pair word), so memory latency overlaps the
// arithmetic of the previous tile.  Compute is the tiled schedule above with
// every tap unrolled (ds_read immediate column offsets).
struct GpPers {
    int32_t xs_n, xs_c, xs_h, xs_w, ys_n, ys_c, ys_h, ys_w;
    int32_t x_bytes, y_bytes;   // buffer ranges of x and y
    int32_t wpg;                // workgroups per group
    uint32_t m_plane, m_iw;     // ceil(2^32 / plane), ceil(2^32 / IW): quotients of operands below 2^16
};

__device__ __forceinline__ int qdiv(int a, uint32_t m) { return (int)__umulhi((uint32_t)a, m); }

template <typename T, int KH, int KW, int P, int JB>
__global__ __launch_bounds__(256) void grp_pers_kernel(GpArgs a, GpPers f)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    constexpr int KK = KH * KW;
    constexpr int ES = Dt<T>::size;
    constexpr int SPT = 8;   // staged words per thread
    constexpr int INVALID = 0x7fffff00;
    uint32_t *sw = smem;                                   // [npairs][KK][cog_pad]
    uint32_t *sx = smem + a.npairs * KK * a.cog_pad;       // [npairs][IH][IW]
    const int tid = threadIdx.x;
    const int g = blockIdx.x % a.G;
    const int tiles = a.N * a.tiles_h * a.tiles_w;
    const int plane = a.IH * a.IW;
    const int words = a.npairs * plane;

    // The group's weights as channel pairs (pad channels zero), once.
    {
        const T *__restrict__ Wt = static_cast<const T *>(a.w);
        for (int i = tid; i < a.npairs * KK * a.cog_pad; i += 256) {
            const int j = i % a.cog_pad;
            const int rest = i / a.cog_pad;
            const int tap = rest % KK;
            const int p = rest / KK;
            uint32_t word = 0;
            if (j < a.Cog) {
                const int64_t base = (int64_t)(g * a.Cog + j) * a.ws0 + (int64_t)(tap / KW) * a.ws2 +
                                     (int64_t)(tap % KW) * a.ws3;
                const uint16_t lo = Wt[base + (int64_t)(2 * p) * a.ws1].u;
                const uint16_t hi = (2 * p + 1 < a.Cig) ? Wt[base + (int64_t)(2 * p + 1) * a.ws1].u : (uint16_t)0;
                word = (uint32_t)lo | ((uint32_t)hi << 16);
            }
            sw[i] = word;
        }
    }

    // This thread's staging slots: word e = tid + 256 k of the tile, i.e.
    // pair e / plane at tile row r, column q; its input offset relative to the
    // tile origin, (r, q), and whether the pair has a second channel.
    int soff[SPT], srq[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int e = tid + 256 * k;
        const int p = qdiv(e, f.m_plane), i = e - p * plane;
        const int r = qdiv(i, f.m_iw), q = i - r * a.IW;
        soff[k] = r * f.xs_h + q * f.xs_w + 2 * p * f.xs_c;
        // bit 31: slot unused; bit 30: no partner channel; then r << 15 | q.
        srq[k] = (e >= words ? (1 << 31) : 0) | (2 * p + 1 >= a.Cig ? (1 << 30) : 0) | (r << 15) | q;
    }
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, f.x_bytes, 0x00020000);
    uint32_t lo[SPT], hi[SPT];
    auto fetch = [&](int j) {
        int t = j;
        const int tw = t % a.tiles_w;
        t /= a.tiles_w;
        const int th = t % a.tiles_h;
        const int n = t / a.tiles_h;
        const int ih0 = th * a.TH * a.SH - a.PH;
        const int iw0 = tw * a.TW * a.SW - a.PW;
        const int base = n * f.xs_n + g * a.Cig * f.xs_c + ih0 * f.xs_h + iw0 * f.xs_w;
        const bool tok = j < tiles;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int rq = srq[k];
            const int r = (rq >> 15) & 0x7fff, q = rq & 0x7fff;
            const bool ok = tok && rq >= 0 && (unsigned)(ih0 + r) < (unsigned)a.H && (unsigned)(iw0 + q) < (unsigned)a.W;
            const int off = ok ? (base + soff[k]) * ES : INVALID;
            const int off2 = ok && !(rq & (1 << 30)) ? off + f.xs_c * ES : INVALID;
            lo[k] = __builtin_amdgcn_raw_buffer_load_b16(xr, off, 0, 0);
            hi[k] = __builtin_amdgcn_raw_buffer_load_b16(xr, off2, 0, 0);
        }
    };

    const int ty = tid / a.tpr;
    const int tx = tid - ty * a.tpr;
    const bool active = ty < a.TH;
    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, f.y_bytes, 0x00020000);
    int xa[KH][P];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int p = 0; p < P; ++p) xa[kh][p] = (ty * a.SH + kh) * a.IW + (tx + p * a.tpr) * a.SW;

    int j = blockIdx.x / a.G;
    fetch(j);
    for (; j < tiles; j += f.wpg) {
        // Stage the fetched tile, then start fetching the next one.
        __syncthreads();   // every thread is done reading the previous tile
#pragma unroll
        for (int k = 0; k < SPT; ++k)
            if (srq[k] >= 0) sx[tid + 256 * k] = (lo[k] & 0xffffu) | (hi[k] << 16);
        __syncthreads();
        int t = j;
        const int tw = t % a.tiles_w;
        t /= a.tiles_w;
        const int th = t % a.tiles_h;
        const int n = t / a.tiles_h;
        fetch(j + f.wpg);

        const int oh = th * a.TH + ty;
        const int ow0 = tw * a.TW + tx;
        if (!active || oh >= a.OH || ow0 >= a.OW) continue;
        const int ybase = n * f.ys_n + oh * f.ys_h + ow0 * f.ys_w;
        for (int j0 = 0; j0 < a.Cog; j0 += JB) {
            float acc[P][JB];
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const float bv = (a.has_bias && j0 + jj < a.Cog) ? to_f32(Bp[g * a.Cog + j0 + jj]) : 0.f;
#pragma unroll
                for (int p = 0; p < P; ++p) acc[p][jj] = bv;
            }
            for (int pr = 0; pr < a.npairs; ++pr) {
                const uint32_t *sxp = sx + pr * plane;
                const uint32_t *swp = sw + pr * KK * a.cog_pad + j0;
#pragma unroll
                for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                    for (int kw = 0; kw < KW; ++kw) {
                        uint32_t xv[P];
#pragma unroll
                        for (int p = 0; p < P; ++p) xv[p] = sxp[xa[kh][p] + kw];
                        const uint32_t *wrow = swp + (kh * KW + kw) * a.cog_pad;
                        uint32_t wv[JB];
#pragma unroll
                        for (int jj = 0; jj < JB; jj += 4) {
                            const uint4 qv = *reinterpret_cast<const uint4 *>(wrow + jj);
                            wv[jj] = qv.x;
                            wv[jj + 1] = qv.y;
                            wv[jj + 2] = qv.z;
                            wv[jj + 3] = qv.w;
                        }
#pragma unroll
                        for (int p = 0; p < P; ++p)
#pragma unroll
                            for (int jj = 0; jj < JB; ++jj) acc[p][jj] = dot2<T>(xv[p], wv[jj], acc[p][jj]);
                    }
            }
            // 16-bit buffer stores at 32-bit offsets; absent columns and
            // channels get an out-of-range vector offset (dropped) -- the
            // scalar offset, which the range check does not cover, stays a
            // real channel offset.
            int yo[P];
#pragma unroll
            for (int p = 0; p < P; ++p)
                yo[p] = ow0 + p * a.tpr < a.OW ? (ybase + (g * a.Cog + j0) * f.ys_c + p * a.tpr * f.ys_w) * ES
                                               : 0x7fffff00;
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const bool cok = j0 + jj < a.Cog;
#pragma unroll
                for (int p = 0; p < P; ++p)
                    __builtin_amdgcn_raw_buffer_store_b16(from_f32<T>(acc[p][jj]).u, yr, cok ? yo[p] : 0x7fffff00,
                                                          cok ? jj * f.ys_c * ES : 0, 0);
            }
        }
    }
}

// Flat schedule (no LDS input tile, no barrier after the weights): thread =
// (image, strip of R output rows, output column) of one group, columns
// fastest, so a wave's loads and stores run along rows.  A workgroup serves
// 256 consecutive threads of one group; the group's weights are staged once
// as channel-pair words in the order [channel block of 8][pair][tap][8], so
// the 8 output channels of one (pair, tap) are two 16-byte LDS broadcasts at
// a compile-time offset from the pair's base.  For each pair the thread loads
// its whole input window -- ((R-1)*S + KH) rows x KW columns, as channel-pair
// words assembled from two 16-bit buffer loads -- with out-of-range rows and
// columns (the padding) and a missing partner channel answered with zeros by
// the buffer range check; the next pair's window is in flight while the
// current one is multiplied.  Each (kh, kw) then feeds R x 8 dot2 from
// registers.  Only the per-lane base offset is a vector offset; pair, row,
// column, channel and output-row offsets are uniform and ride in the scalar
// offset (not range-checked, and only ever added to a valid base).
struct GpFlat {
    int32_t xs_n, xs_c, xs_h, xs_w, ys_n, ys_c, ys_h, ys_w;
    int32_t x_bytes, y_bytes;   // buffer ranges of x and y
    int32_t strips;             // ceil(OH / R)
    int32_t per_group;          // threads per group: N * strips * OW
    int32_t wpg;                // workgroups per group
    int32_t nblk;               // channel blocks of 8: cog_pad / 8
    int32_t x_lead;             // bytes of the largest negative window offset: (PH * xs_h + PW * xs_w) * ES
};

template <typename T, int KH, int KW, int S, int R>
__global__ __launch_bounds__(256) void grp_flat_kernel(GpArgs a, GpFlat f)
{
    constexpr int ES = Dt<T>::size;
    constexpr int KK = KH * KW;
    constexpr int NR = (R - 1) * S + KH;            // window rows
    constexpr int WIN = NR * KW;                    // window words per pair
    constexpr bool PREF = 2 * WIN <= 64;            // double-buffer the window
    constexpr int INVALID = 0x7fffff00;
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];   // [nblk][npairs][KK][8]

    const int tid = threadIdx.x;
    const int g = blockIdx.x / f.wpg;
    const int q = (blockIdx.x - g * f.wpg) * 256 + tid;
    const int np = a.npairs;

    {
        const T *__restrict__ Wt = static_cast<const T *>(a.w);
        const int total = f.nblk * np * KK * 8;
        for (int e = tid; e < total; e += 256) {
            const int jj = e & 7;
            int r = e >> 3;
            const int tap = r % KK;
            r /= KK;
            const int p = r % np;
            const int jb = r / np;
            const int j = jb * 8 + jj;
            uint32_t word = 0;
            if (j < a.Cog) {
                const int64_t base = (int64_t)(g * a.Cog + j) * a.ws0 + (int64_t)(tap / KW) * a.ws2 +
                                     (int64_t)(tap % KW) * a.ws3;
                const uint16_t lo = Wt[base + (int64_t)(2 * p) * a.ws1].u;
                const uint16_t hi = (2 * p + 1 < a.Cig) ? Wt[base + (int64_t)(2 * p + 1) * a.ws1].u : (uint16_t)0;
                word = (uint32_t)lo | ((uint32_t)hi << 16);
            }
            smem[e] = word;
        }
    }
    __syncthreads();
    if (q >= f.per_group) return;

    const int ow = q % a.OW;
    const int t = q / a.OW;
    const int strip = t % f.strips;
    const int n = t / f.strips;
    const int oh0 = strip * R;
    const int ih0 = oh0 * (R == 1 ? a.SH : S) - a.PH;
    const int iw0 = ow * S - a.PW;

    // Per-lane base offset of the window origin (row ih0, column iw0), or
    // the out-of-range marker for rows outside the input; a column outside it
    // replaces the base by the marker at its loads.  The origin lies up to
    // f.x_lead bytes before x (the padding before), so x is addressed from a
    // base that many bytes lower: every base offset is then non-negative.
    const int xbase = f.x_lead + (n * f.xs_n + g * a.Cig * f.xs_c + ih0 * f.xs_h + iw0 * f.xs_w) * ES;
    int vrow[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) vrow[i] = (unsigned)(ih0 + i) < (unsigned)a.H ? xbase : INVALID;
    bool cok[KW];
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) cok[kw] = (unsigned)(iw0 + kw) < (unsigned)a.W;

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char *>(static_cast<const unsigned char *>(a.x)) - f.x_lead, (short)0,
        f.x_bytes + f.x_lead, 0x00020000);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, f.y_bytes, 0x00020000);

    // Vector offsets of the window's loads: fixed for the thread, so kept
    // in registers when the window is small (recomputed per load otherwise).
    int vo_keep[PREF ? WIN : 1];
    if constexpr (PREF) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int kw = 0; kw < KW; ++kw) vo_keep[i * KW + kw] = cok[kw] ? vrow[i] : INVALID;
    }
    auto vo_at = [&](int i, int kw) {
        if constexpr (PREF) return vo_keep[i * KW + kw];
        else return cok[kw] ? vrow[i] : INVALID;
    };
    // Pair p's window; a pair without a second channel (odd Cig) leaves the
    // high halves zero.  Pair, row and column offsets are uniform: scalar.
    const bool odd = a.Cig & 1;
    auto load_window = [&](int p, uint32_t (&xw)[WIN]) {
        const int sp = 2 * p * f.xs_c * ES;
        if (!odd || 2 * p + 1 < a.Cig) {
#pragma unroll
            for (int i = 0; i < NR; ++i)
#pragma unroll
                for (int kw = 0; kw < KW; ++kw) {
                    const int vo = vo_at(i, kw);
                    const int so = sp + (i * f.xs_h + kw * f.xs_w) * ES;
                    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(xr, vo, so, 0);
                    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(xr, vo, so + f.xs_c * ES, 0);
                    xw[i * KW + kw] = lo | (hi << 16);
                }
        } else {
#pragma unroll
            for (int i = 0; i < NR; ++i)
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
                    xw[i * KW + kw] = __builtin_amdgcn_raw_buffer_load_b16(
                        xr, vo_at(i, kw), sp + (i * f.xs_h + kw * f.xs_w) * ES, 0);
        }
    };

    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    int yo[R];
    const int ybase = (n * f.ys_n + g * a.Cog * f.ys_c + oh0 * f.ys_h + ow * f.ys_w) * ES;
#pragma unroll
    for (int r = 0; r < R; ++r) yo[r] = oh0 + r < a.OH ? ybase : INVALID;

    for (int jb = 0; jb < f.nblk; ++jb) {
        float acc[R][8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int j = jb * 8 + jj;
            const float bv = (a.has_bias && j < a.Cog) ? to_f32(Bp[g * a.Cog + j]) : 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][jj] = bv;
        }
        auto compute = [&](int p, const uint32_t (&xw)[WIN]) {
            const uint32_t *wp = smem + (jb * np + p) * KK * 8;
#pragma unroll
            for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                for (int kw = 0; kw < KW; ++kw) {
                    const uint4 w0 = *reinterpret_cast<const uint4 *>(wp + (kh * KW + kw) * 8);
                    const uint4 w1 = *reinterpret_cast<const uint4 *>(wp + (kh * KW + kw) * 8 + 4);
                    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t xv = xw[(r * S + kh) * KW + kw];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) acc[r][jj] = dot2<T>(xv, wv[jj], acc[r][jj]);
                    }
                }
        };
        uint32_t xa[WIN];
        load_window(0, xa);
        if constexpr (PREF) {
            // Pairs alternate between two windows; the next pair's window is
            // issued before the current one is multiplied.
            uint32_t xb[WIN];
            for (int p = 0; p < np; p += 2) {
                if (p + 1 < np) load_window(p + 1, xb);
                compute(p, xa);
                if (p + 1 < np) {
                    if (p + 2 < np) load_window(p + 2, xa);
                    compute(p + 1, xb);
                }
            }
        } else {
            for (int p = 0; p < np; ++p) {
                compute(p, xa);
                if (p + 1 < np) load_window(p + 1, xa);
            }
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int j = jb * 8 + jj;
            if (j >= a.Cog) break;
#pragma unroll
            for (int r = 0; r < R; ++r)
                __builtin_amdgcn_raw_buffer_store_b16(from_f32<T>(acc[r][jj]).u, yr, yo[r],
                                                      (j * f.ys_c + r * f.ys_h) * ES, 0);
        }
    }
}

// Plane schedule for 3x3 calls whose groups are whole NCHW planes.  The
// group's Cig input planes are one contiguous run of x and its Cog output
// planes one contiguous run of y, so inputs arrive with 16-byte loads and
// outputs leave with 8-byte stores (a handful of instructions per thread,
// whole cache lines).  Workgroup w serves group w mod G for the images
// w / G, w / G + wpg, ...: its lanes keep their channel's weights in
// registers for every image, and the next image's input chunk is in flight
// into registers while the current image is multiplied.  In LDS the input is
// channel-pair words with a zero halo, [pair][row][column] (the halo and the
// partner of an odd channel are zeroed once and never written), and the
// output is staged as stored values, [channel][row][column].  Thread =
// (output channel j, block of RB rows x CB columns), j fastest: the lanes of
// one block read the same input words (an LDS broadcast).  The block's input
// rows are streamed once; each row feeds the RB x CB accumulators of every
// output row whose window covers it, v_dot2_f32 over both channels of a pair.
struct GpLds {
    int32_t xs_n, ys_n;          // image strides, elements
    int32_t x_bytes, y_bytes;    // buffer ranges
    int32_t IHh, IWh;            // haloed input plane: (OH-1)*S + 3 rows, (OW-1)*S + 3 columns
    int32_t nrb, ncb;            // row / column blocks of the output plane
    int32_t in_words;            // NP * IHh * IWh rounded up to 4
    int32_t out_off;             // LDS byte offset of the output staging
    int32_t chunks_in;           // 16-byte chunks of one group's input planes
    int32_t pieces_out;          // 8-byte pieces of one group's output planes
    int32_t wpg;                 // workgroups per group
};

template <typename T, int NP, int S, int RB, int CB>
__global__ __launch_bounds__(512) void grp_lds_kernel(GpArgs a, GpLds f)
{
    constexpr int ES = Dt<T>::size;
    constexpr int K = 3, KK = 9;
    constexpr int NRW = (RB - 1) * S + K;       // input rows of a block
    constexpr int NCW = (CB - 1) * S + K;       // input columns of a block
    constexpr int INVALID = 0x7fffff00;
    constexpr int OUT_IT = 4;                   // 8-byte output pieces per thread (pieces_out <= 4 * threads)
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    uint32_t *sin = smem;
    unsigned char *sout = reinterpret_cast<unsigned char *>(smem) + f.out_off;

    const int tid = threadIdx.x, nt = blockDim.x;
    const int g = blockIdx.x % a.G;
    const int HW = a.H * a.W;
    const int item = a.Cig * HW;                          // input elements of the group

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, f.x_bytes, 0x00020000);
    const bool has_chunk = tid < f.chunks_in;
    const int xoff0 = (g * item) * ES + tid * 16;
    auto fetch = [&](int n) {
        const bool ok = has_chunk && n < a.N;
        return __builtin_bit_cast(u32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? xoff0 + n * f.xs_n * ES : INVALID, 0, 0));
    };
    int n = blockIdx.x / a.G;
    u32x4 chunk = fetch(n);

    // LDS byte address of each element of this thread's chunk (channel c,
    // row h, column w -> its half of pair word (c/2, h + PH, w + PW)), or -1
    // for elements past the group or outside the haloed plane.
    int saddr[8];
    {
        const int e0 = tid * 8;
        int c = e0 / HW;
        const int rem = e0 - c * HW;
        int h = rem / a.W;
        int w = rem - h * a.W;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int hh = h + a.PH, ww = w + a.PW;
            saddr[k] = (has_chunk && e0 + k < item && hh < f.IHh && ww < f.IWh)
                           ? (((c >> 1) * f.IHh + hh) * f.IWh + ww) * 4 + (c & 1) * 2
                           : -1;
            if (++w == a.W) {
                w = 0;
                if (++h == a.H) {
                    h = 0;
                    ++c;
                }
            }
        }
    }

    // Zero the input plane once: the halo and the partner halves of an odd
    // channel count are never written afterwards.
    for (int i = tid * 4; i < f.in_words; i += nt * 4)
        *reinterpret_cast<u32x4 *>(sin + i) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    const int j = tid % a.Cog;
    const int blk = tid / a.Cog;
    const bool active = blk < f.nrb * f.ncb;
    const int rb = blk / f.ncb, cb = blk - rb * f.ncb;
    // This lane's weights as channel-pair words (missing channels zero).
    uint32_t wr[NP][KK];
    float bv = 0.f;
    {
        const T *__restrict__ Wt = static_cast<const T *>(a.w);
        const int64_t wbase = (int64_t)(g * a.Cog + (active ? j : 0)) * a.ws0;
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int t = 0; t < KK; ++t) {
                const int64_t o = wbase + (int64_t)(t / K) * a.ws2 + (int64_t)(t % K) * a.ws3;
                const uint32_t lo = 2 * p < a.Cig ? Wt[o + (int64_t)(2 * p) * a.ws1].u : 0u;
                const uint32_t hi = 2 * p + 1 < a.Cig ? Wt[o + (int64_t)(2 * p + 1) * a.ws1].u : 0u;
                wr[p][t] = lo | (hi << 16);
            }
        const T *__restrict__ Bp = static_cast<const T *>(a.b);
        if (a.has_bias && active) bv = to_f32(Bp[g * a.Cog + j]);
    }
    const uint32_t *src = sin + (rb * RB * S) * f.IWh + cb * CB * S;
    const int plane = f.IHh * f.IWh;
    uint16_t *so = reinterpret_cast<uint16_t *>(sout) + j * a.OH * a.OW;
    uint16_t *spare = reinterpret_cast<uint16_t *>(sout + f.pieces_out * 8);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, f.y_bytes, 0x00020000);
    const int yoff0 = g * a.Cog * a.OH * a.OW * ES;

    for (; n < a.N; n += f.wpg) {
        // The previous image's multiply finished before its last barrier:
        // the input plane is free.  Scatter this image's chunk, then fetch
        // the next one into the same registers.
        unsigned char *sb = reinterpret_cast<unsigned char *>(sin);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (saddr[k] >= 0) {
                const uint32_t word = chunk[k >> 1];
                *reinterpret_cast<uint16_t *>(sb + saddr[k]) = (k & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
            }
        chunk = fetch(n + f.wpg);
        __syncthreads();

        if (active) {
            float acc[RB][CB];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr)
#pragma unroll
                for (int cc = 0; cc < CB; ++cc) acc[rr][cc] = bv;
#pragma unroll
            for (int i = 0; i < NRW; ++i) {
                uint32_t xw[NP][NCW];
#pragma unroll
                for (int p = 0; p < NP; ++p)
#pragma unroll
                    for (int c = 0; c < NCW; ++c) xw[p][c] = src[p * plane + i * f.IWh + c];
#pragma unroll
                for (int rr = 0; rr < RB; ++rr) {
                    const int kh = i - rr * S;
                    if (kh < 0 || kh >= K) continue;
#pragma unroll
                    for (int kw = 0; kw < K; ++kw)
#pragma unroll
                        for (int p = 0; p < NP; ++p)
#pragma unroll
                            for (int cc = 0; cc < CB; ++cc)
                                acc[rr][cc] = dot2<T>(xw[p][cc * S + kw], wr[p][kh * K + kw], acc[rr][cc]);
                }
            }
            // Stage the rounded outputs of the block, [j][oh][ow]; positions
            // past the plane go to a spare slot after the staging area.  The
            // previous image's staged outputs were read before the barrier
            // above.
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const int oh = rb * RB + rr;
#pragma unroll
                for (int cc = 0; cc < CB; ++cc) {
                    const int ow = cb * CB + cc;
                    const bool ok = oh < a.OH && ow < a.OW;
                    uint16_t *dst = ok ? so + oh * a.OW + ow : spare;
                    *dst = from_f32<T>(acc[rr][cc]).u;
                }
            }
        }
        __syncthreads();

        // The group's output planes of image n are one contiguous run of y:
        // OUT_IT 8-byte pieces per thread (the last ones dropped by the
        // range check).  The stores are ordinary compiler-visible stores of
        // at most 8 bytes, a fixed number of them, so the next image's wait
        // for its input chunk need not wait for them as well.
        const int yoff = yoff0 + n * f.ys_n * ES;
#pragma unroll
        for (int r = 0; r < OUT_IT; ++r) {
            const int q = tid + r * nt;
            const bool ok = q < f.pieces_out;
            typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
            const u32x2 v = *reinterpret_cast<const u32x2 *>(sout + (ok ? q : 0) * 8);
            __builtin_amdgcn_raw_buffer_store_b64(v, yr, ok ? yoff + q * 8 : INVALID, 0, kStoreNT);
        }
    }
}

// Grouped 3x3 calls whose groups are whole NCHW planes, on the matrix cores.
// Per group the convolution is a small dense contraction,
//   Y[position, j] = sum over (tap t, channel c) of X[position + t, c] * W[t, c, j],
// with K = 9 taps x CP channel slots (CP = Cig rounded up to 4 or 8) and
// N = Cog <= 16.  Workgroup w serves group w mod G for the images w / G,
// w / G + wpg, ...; its lanes keep the weights (the MFMA B operand) in
// registers, and the next image's input chunks are in flight into registers
// while the current image is multiplied.  The group's input planes (one
// contiguous run of x) arrive with 16-byte loads and are scattered into an
// LDS plane with a zero halo in position-major order, [row][column][CP
// channels], so the 8 consecutive K elements a lane feeds to one
// v_mfma_f32_16x16x32 are 2 taps x 4 channels (CP = 4) or 1 tap x 8 channels
// (CP = 8) of one position: one 8- or 16-byte LDS read.  An MFMA tile is 16
// consecutive output columns of one output row (the last tile of a row
// partly idle); K runs over ceil(9 CP / 32) steps, and the lanes whose K
// slice lies past the ninth tap feed zeros.  Accumulators start from the
// bias; each lane ends with 4 consecutive columns of one output channel,
// rounded once and
// staged in LDS as [channel][row][column]; the group's contiguous output
// planes then leave as 8-byte pieces.
struct GpMma {
    int32_t xs_n, ys_n;          // image strides, elements
    int32_t x_bytes, y_bytes;    // buffer ranges
    int32_t IHh, IWh;            // haloed input plane: (OH-1)*S + 3 rows, (OW-1)*S + 3 columns
    int32_t in_bytes;            // bytes of the LDS input plane, a multiple of 16
    int32_t chunks_in;           // 16-byte chunks of one group's input planes
    int32_t pieces_out;          // 8-byte pieces of one group's output planes
    int32_t ctiles;              // 16-column tiles per output row
    uint32_t m_ct;               // ceil(2^32 / ctiles) for ctiles >= 2: quotients of tile indices below 2^16
    int32_t wpg;                 // workgroups per group
};

template <typename T, int CP, int S, bool PM>
__global__ __launch_bounds__(256) void grp_mma_kernel(GpArgs a, GpMma f)
{
    constexpr int ES = Dt<T>::size;
    constexpr int KS = (9 * CP + 31) / 32;      // MFMA K steps
    constexpr int IN_IT = PM ? CP : 2;          // chunks per thread (host-checked)
    constexpr int OUT_IT = 8;                   // output pieces per thread (host-checked)
    constexpr int INVALID = 0x7fffff00;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *sin = lds;                   // [IHh][IWh][CP] stored values
    unsigned char *sout = lds + f.in_bytes;     // [Cog][OH][OW] stored values

    const int tid = threadIdx.x;
    // The wave index is uniform: in a scalar register, so tile arithmetic
    // stays scalar.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = blockIdx.x % a.G;
    const int HW = a.H * a.W;
    const int OHW = a.OH * a.OW;
    const int item = a.Cig * HW;

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, f.x_bytes, 0x00020000);
    // PM (planes of whole 16-byte chunks, HW / 8 <= 256): thread t < HW / 8
    // loads the 8 positions 8t .. 8t + 7 of every channel (chunk c = channel
    // c), so it holds each position's channels together and writes them to
    // LDS as one 8- or 16-byte vector.  Otherwise chunk r of thread t is the
    // group's 16-byte chunk t + 256 r, whose 8 elements go to LDS one by one.
    const int xoff0 = g * item * ES + tid * 16;
    u32x4 chunk[IN_IT];
    auto fetch = [&](int n) {
#pragma unroll
        for (int r = 0; r < IN_IT; ++r) {
            const bool ok = PM ? n < a.N && tid * 8 < HW && r < a.Cig : n < a.N && tid + r * 256 < f.chunks_in;
            const int off = PM ? xoff0 + r * HW * ES : xoff0 + r * 256 * 16;
            chunk[r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? off + n * f.xs_n * ES : INVALID, 0, 0));
        }
    };
    int n = blockIdx.x / a.G;
    fetch(n);

    // LDS byte address of each element of this thread's chunks (channel c,
    // row h, column w -> slot c of position (h + PH, w + PW)), or -1 for
    // elements past the group or outside the haloed plane.
    constexpr int SR = PM ? 1 : IN_IT;          // chunk rows with their own addresses
    int saddr[SR][8];
#pragma unroll
    for (int r = 0; r < SR; ++r) {
        const int e0 = (tid + r * 256) * 8;
        int c = e0 / HW;
        const int rem = e0 - c * HW;
        int h = rem / a.W;
        int w = rem - h * a.W;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int hh = h + a.PH, ww = w + a.PW;
            const int lim = PM ? HW : item;
            saddr[r][k] = (e0 + k < lim && hh < f.IHh && ww < f.IWh) ? ((hh * f.IWh + ww) * CP + c) * ES : -1;
            if (++w == a.W) {
                w = 0;
                if (++h == a.H) {
                    h = 0;
                    ++c;
                }
            }
        }
    }

    // Weights as the MFMA B operand: lane l holds K elements
    // 32 s + 8 (l / 16) + i of output channel l % 16, K = tap * CP + channel
    // (zero past the ninth tap, past Cig and past Cog).
    const int jn = lane & 15, kq = lane >> 4;
    uint4 bw[KS];
    {
        const T *__restrict__ Wt = static_cast<const T *>(a.w);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint16_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = s * 32 + kq * 8 + i;
                const int t = k / CP, c = k % CP;
                const bool ok = jn < a.Cog && t < 9 && c < a.Cig;
                const int64_t o = ok ? (int64_t)(g * a.Cog + jn) * a.ws0 + (int64_t)c * a.ws1 +
                                           (int64_t)(t / 3) * a.ws2 + (int64_t)(t % 3) * a.ws3
                                     : 0;
                const uint16_t v = Wt[o].u;
                h[i] = ok ? v : (uint16_t)0;
            }
            __builtin_memcpy(&bw[s], h, 16);
        }
    }
    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    const float bias = (a.has_bias && jn < a.Cog) ? to_f32(Bp[g * a.Cog + jn]) : 0.f;

    // Per-lane LDS offsets of the K slices (relative to the position's
    // window origin): CP = 4 reads taps t0 and t0 + 1, CP = 8 tap t; a tap
    // past the ninth reads nothing (zeros).
    int toff[KS][2];
    bool tok[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = CP == 4 ? 8 * s + 2 * kq + u : 4 * s + kq;
            tok[s][u] = t < 9 && (CP == 4 || u == 0);
            toff[s][u] = ((t / 3) * f.IWh + t % 3) * CP * ES;
        }
    }

    // Zero the input plane once: the halo and the channel slots past Cig are
    // never written afterwards.
    for (int i = tid * 16; i < f.in_bytes; i += 256 * 16)
        *reinterpret_cast<u32x4 *>(sin + i) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    // Tiles: (output row, 16-column block), wave w takes tiles w, w + 4, ...
    const int ntiles = a.OH * f.ctiles;
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, f.y_bytes, 0x00020000);
    const int yoff0 = g * a.Cog * OHW * ES + tid * 8;
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

    for (; n < a.N; n += f.wpg) {
        // The previous image's tiles were read before its last barrier: the
        // plane is free.  Scatter this image's chunks, fetch the next ones.
        if constexpr (PM) {
            // Position k of the thread's block: its CP channel values, low
            // or high halves of word k / 2 of each chunk, paired by one byte
            // permute per two channels.
            const uint32_t sel = 0x05040100u;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (saddr[0][k] < 0) continue;
                const uint32_t sk = (k & 1) ? sel + 0x02020202u : sel;
                uint32_t wv[CP / 2];
#pragma unroll
                for (int q = 0; q < CP / 2; ++q)
                    wv[q] = __builtin_amdgcn_perm(chunk[2 * q + 1][k >> 1], chunk[2 * q][k >> 1], sk);
                if constexpr (CP == 4)
                    *reinterpret_cast<uint2 *>(sin + saddr[0][k]) = uint2{wv[0], wv[1]};
                else
                    *reinterpret_cast<uint4 *>(sin + saddr[0][k]) = uint4{wv[0], wv[1], wv[2], wv[3]};
            }
        } else {
#pragma unroll
            for (int r = 0; r < IN_IT; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (saddr[r][k] >= 0) {
                        const uint32_t word = chunk[r][k >> 1];
                        *reinterpret_cast<uint16_t *>(sin + saddr[r][k]) =
                            (k & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
                    }
        }
        fetch(n + f.wpg);
        __syncthreads();

        // Two independent tiles per pass (w and w + 4), so their LDS reads,
        // MFMAs and stores overlap; a tile past the plane repeats the last one
        // and keeps nothing.  (Four per pass measured 5% slower: the extra
        // registers cost a resident workgroup per CU.)
        constexpr int TU = 2;
        for (int t0 = wave; t0 < ntiles; t0 += 4 * TU) {
            f32x4 acc[TU];
            uint4 av[TU][KS];
            int oh[TU], ow0[TU];
#pragma unroll
            for (int u = 0; u < TU; ++u) {
                const int tile = min(t0 + 4 * u, ntiles - 1);
                // tile / ctiles (tile < 2^16; one tile per row needs no division)
                oh[u] = f.ctiles == 1 ? tile : (int)__umulhi((uint32_t)tile, f.m_ct);
                ow0[u] = (tile - oh[u] * f.ctiles) * 16;
                const int ow = min(ow0[u] + (lane & 15), a.OW - 1);
                const unsigned char *base = sin + ((oh[u] * S) * f.IWh + ow * S) * CP * ES;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    av[u][s] = uint4{0u, 0u, 0u, 0u};
                    if constexpr (CP == 4) {
                        uint2 lo = {0u, 0u}, hi = {0u, 0u};
                        if (tok[s][0]) lo = *reinterpret_cast<const uint2 *>(base + toff[s][0]);
                        if (tok[s][1]) hi = *reinterpret_cast<const uint2 *>(base + toff[s][1]);
                        av[u][s] = uint4{lo.x, lo.y, hi.x, hi.y};
                    } else {
                        if (tok[s][0]) av[u][s] = *reinterpret_cast<const uint4 *>(base + toff[s][0]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < TU; ++u) {
                acc[u] = f32x4{bias, bias, bias, bias};
#pragma unroll
                for (int s = 0; s < KS; ++s) mma_16x16x32(av[u][s], bw[s], acc[u], T{});
            }
#pragma unroll
            for (int u = 0; u < TU; ++u) {
                // Lane l holds columns ow0 + 4 (l / 16) + i of channel l % 16
                // (OW % 4 == 0: all four columns valid or none).
                const int oc = ow0[u] + 4 * kq;
                // Lanes past Cog (or past the plane) store nothing: a shared
                // spare slot would put every one of them on one LDS bank.
                const bool keep = jn < a.Cog && oc < a.OW && t0 + 4 * u < ntiles;
                if (keep) {
                    uint2 v;
                    v.x = pack2<T>(acc[u][0], acc[u][1]);
                    v.y = pack2<T>(acc[u][2], acc[u][3]);
                    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(sout) + (jn * a.OH + oh[u]) * a.OW + oc) = v;
                }
            }
        }
        __syncthreads();

        // The group's output planes of image n are one contiguous run of y:
        // a fixed number of compiler-visible 8-byte stores per thread, so the
        // next image's wait for its chunks need not wait for them.
        const int yoff = yoff0 + n * f.ys_n * ES;
#pragma unroll
        for (int r = 0; r < OUT_IT; ++r) {
            const int q = tid + r * 256;
            const bool ok = q < f.pieces_out;
            const u32x2 v = *reinterpret_cast<const u32x2 *>(sout + (ok ? q : 0) * 8);
            __builtin_amdgcn_raw_buffer_store_b64(v, yr, ok ? yoff + r * 256 * 8 : INVALID, 0, kStoreNT);
        }
    }
}

namespace {
constexpr int kP = 4;
constexpr int kJB = 8;
constexpr int64_t kLds = 64 * 1024;
}  // namespace

// Shape and stride conditions of the matrix-core plane schedule (pointer
// alignment is checked at launch): 2-D 3x3, equal strides 1 or 2, unit
// dilation, at most 16 output channels per group, NCHW-contiguous group
// planes in whole 16-byte (input) and 8-byte (output) pieces, output rows of
// a multiple of 4 columns, the fixed per-thread load / store counts and the
// LDS budget, 32-bit offsets.
bool grp_mma_plane_ok(const conv_desc &d, const conv_tensor &y)
{
    if (d.spatial != 2 || d.dtype == CONV_F32 || d.transposed) return false;
    const int64_t Cig = d.C_in / d.groups, Cog = d.C_out / d.groups;
    if (d.k[0] != 3 || d.k[1] != 3 || d.stride[0] != d.stride[1] || (d.stride[0] != 1 && d.stride[0] != 2) ||
        d.dilation[0] != 1 || d.dilation[1] != 1 || Cig > 8 || Cog > 16)
        return false;
    const int64_t es = esize(d.dtype);
    const int64_t H = d.in[0], W = d.in[1], OH = d.out[0], OW = d.out[1], S = d.stride[0];
    const int64_t OHW = OH * OW;
    const int64_t in_bytes = Cig * H * W * es, out_bytes = Cog * OHW * es;
    const int64_t CP = Cig <= 4 ? 4 : 8;
    const int64_t lds_total = round_up(((OH - 1) * S + 3) * ((OW - 1) * S + 3) * CP * es, 16) + round_up(out_bytes, 16) + 16;
    const bool xdense = d.x.strides[3] == 1 && d.x.strides[2] == W && d.x.strides[1] == H * W &&
                        (d.x.strides[0] * es) % 16 == 0 && in_bytes % 16 == 0;
    const bool ydense = y.strides[3] == 1 && y.strides[2] == OW && y.strides[1] == OHW && (y.strides[0] * es) % 8 == 0 &&
                        out_bytes % 8 == 0;
    auto span = [&](const conv_tensor &t) {
        int64_t o = 0;
        for (int i = 0; i < t.rank; ++i)
            if (t.sizes[i] > 0) o += (t.sizes[i] - 1) * t.strides[i];
        return (o + 1) * es;
    };
    const int64_t lim = 0x7fffffffLL - 4096;
    return xdense && ydense && OW % 4 == 0 && in_bytes / 16 <= 2 * 256 && out_bytes / 8 <= 8 * 256 &&
           OH * cdiv(OW, 16) < 65536 && lds_total <= kLds && span(d.x) < lim && span(y) < lim &&
           d.N * d.groups < (1LL << 31);
}

bool grp_supported(const conv_desc &d)
{
    if (d.dtype == CONV_F32 || d.transposed) return false;
    if (d.spatial != 1 && d.spatial != 2) return false;
    const int64_t cig = d.C_in / d.groups;
    return cig >= 1 && cig <= 8;
}

// LDS of the tiled schedule's smallest tile (one output row of kP columns):
// the group's weights (input-channel pairs x taps x padded outputs, one word
// each) plus the halo rows.  Every grouped schedule stages the weights.
static int64_t grp_min_lds(const conv_desc &d)
{
    const bool two = d.spatial == 2;
    const int64_t KH = two ? d.k[0] : 1, KW = two ? d.k[1] : d.k[0];
    const int64_t SW = two ? d.stride[1] : d.stride[0];
    const int64_t DW = two ? d.dilation[1] : d.dilation[0];
    const int64_t DH = two ? d.dilation[0] : 1;
    const int64_t npairs = (d.C_in / d.groups + 1) / 2;
    const int64_t cog_pad = round_up(d.C_out / d.groups, kJB);
    const int64_t ih = (KH - 1) * DH + 1, iw = (kP - 1) * SW + (KW - 1) * DW + 1;
    return 4 * (npairs * KH * KW * cog_pad + npairs * ih * iw);
}

bool grp_fits(const conv_desc &d) { return grp_min_lds(d) <= kLds; }

bool grp_geometry(const conv_desc &d, conv_plan_t &p)
{
    if (!grp_fits(d)) return false;
    const bool two = d.spatial == 2;
    const int64_t OH = two ? d.out[0] : 1, OW = two ? d.out[1] : d.out[0];
    const int64_t KH = two ? d.k[0] : 1, KW = two ? d.k[1] : d.k[0];
    const int64_t SH = two ? d.stride[0] : 1, SW = two ? d.stride[1] : d.stride[0];
    const int64_t DH = two ? d.dilation[0] : 1, DW = two ? d.dilation[1] : d.dilation[0];
    const int64_t npairs = (d.C_in / d.groups + 1) / 2;
    const int64_t cog_pad = round_up(d.C_out / d.groups, kJB);
    int64_t TW = OW < kP * 64 ? round_up(OW, kP) : kP * 64;
    int64_t tpr = TW / kP;
    int64_t TH = 256 / tpr;
    auto lds = [&](int64_t th, int64_t tw) {
        const int64_t ih = (th - 1) * SH + (KH - 1) * DH + 1;
        const int64_t iw = (tw - 1) * SW + (KW - 1) * DW + 1;
        return 4 * (npairs * KH * KW * cog_pad + npairs * ih * iw);
    };
    while (TH > 1 && lds(TH, TW) > kLds) TH /= 2;
    while (TW > kP && lds(TH, TW) > kLds) {
        TW = round_up(TW / 2, kP);
        tpr = TW / kP;
    }
    if (TH > OH) TH = OH;
    p.tile[0] = TH;
    p.tile[1] = TW;
    p.tile[2] = tpr;
    p.tile[3] = npairs;
    p.tile[4] = (TH - 1) * SH + (KH - 1) * DH + 1;
    p.tile[5] = (TW - 1) * SW + (KW - 1) * DW + 1;
    p.tile[6] = cdiv(OH, TH);
    p.tile[7] = cdiv(OW, TW);
    p.grid[0] = d.N * d.groups * p.tile[6] * p.tile[7];
    p.block = 256;
    p.lds_bytes = (int32_t)lds(TH, TW);
    p.variant = grp_mma_plane_ok(d, p.y) ? GRP_SCHED_MMA : GRP_SCHED_VALU;
    return p.lds_bytes <= kLds;
}

int launch_grp(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream)
{
    const conv_desc &d = p.d;
    GpArgs a;
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
    auto at = [&](const int64_t *v, int i, int64_t dflt) { return (int32_t)(i < 0 ? dflt : v[i]); };
    a.N = (int32_t)d.N;
    a.G = (int32_t)d.groups;
    a.Cig = (int32_t)(d.C_in / d.groups);
    a.Cog = (int32_t)(d.C_out / d.groups);
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
    a.TH = (int32_t)p.tile[0];
    a.TW = (int32_t)p.tile[1];
    a.tpr = (int32_t)p.tile[2];
    a.npairs = (int32_t)p.tile[3];
    a.IH = (int32_t)p.tile[4];
    a.IW = (int32_t)p.tile[5];
    a.tiles_h = (int32_t)p.tile[6];
    a.tiles_w = (int32_t)p.tile[7];
    a.total = (int32_t)p.grid[0];
    a.has_bias = d.has_bias;
    a.cog_pad = (int32_t)round_up(a.Cog, kJB);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)p.grid[0]), block(256);
    const size_t lds = (size_t)p.lds_bytes;
    // Persistent schedule: unit dilation, a compiled kernel extent, 32-bit
    // offsets, at most 8 staged words per thread.
    const int64_t lim = 0x7fffffffLL - 4096;
    auto span = [&](const conv_tensor &t) {
        int64_t o = 0;
        for (int i = 0; i < t.rank; ++i)
            if (t.sizes[i] > 0) o += (t.sizes[i] - 1) * t.strides[i];
        return o + 1;
    };
    // Matrix-core plane schedule (planned from shapes and strides), when x
    // is 16-byte and y 8-byte aligned.
    if (p.variant == GRP_SCHED_MMA && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(y) & 7) == 0) {
        const int64_t es = esize(d.dtype);
        const int64_t S = a.SH;
        const int64_t CP = a.Cig <= 4 ? 4 : 8;
        const int64_t IHh = (a.OH - 1) * S + 3, IWh = (a.OW - 1) * S + 3;
        const int64_t OHW = (int64_t)a.OH * a.OW;
        const int64_t in_lds = round_up(IHh * IWh * CP * es, 16);
        const int64_t out_bytes = (int64_t)a.Cog * OHW * es;
        const int64_t lds_total = in_lds + round_up(out_bytes, 16) + 16;
        const int64_t in_bytes = (int64_t)a.Cig * a.H * a.W * es;
        {
            GpMma f;
            f.xs_n = (int32_t)a.xs_n;
            f.ys_n = (int32_t)a.ys_n;
            f.x_bytes = (int32_t)(span(d.x) * es);
            f.y_bytes = (int32_t)(span(p.y) * es);
            f.IHh = (int32_t)IHh;
            f.IWh = (int32_t)IWh;
            f.in_bytes = (int32_t)in_lds;
            f.chunks_in = (int32_t)(in_bytes / 16);
            f.pieces_out = (int32_t)(out_bytes / 8);
            f.ctiles = (int32_t)cdiv(a.OW, 16);
            f.m_ct = f.ctiles > 1 ? (uint32_t)(((1ULL << 32) + f.ctiles - 1) / f.ctiles) : 0u;
            int dev = 0, cus = 256;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                cus = 256;
            const size_t mlds = (size_t)lds_total;
            // One resident round of workgroups, spread over the groups.
            auto go = [&](auto kern) {
                int per_cu = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, mlds) != hipSuccess || per_cu < 1)
                    per_cu = 1;
                // As many images per workgroup for every workgroup of a group.
                const int64_t most = std::max<int64_t>(1, std::min<int64_t>(a.N, (int64_t)per_cu * cus / a.G));
                f.wpg = (int32_t)cdiv(a.N, cdiv(a.N, most));
                hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.G * f.wpg)), dim3(256), mlds, s, a, f);
                return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
            };
            // Position-major chunks when every channel plane is whole 16-byte
            // chunks and one thread per 8 positions suffices.
            const int64_t HW = (int64_t)a.H * a.W;
            const bool pm = (HW * es) % 16 == 0 && HW % 8 == 0 && HW / 8 <= 256;
#define MICONV_GM(CP_, S_)                                                                             \
    if (CP == CP_ && S == S_) {                                                                        \
        if (pm)                                                                                        \
            return d.dtype == CONV_F16 ? go(grp_mma_kernel<f16_t, CP_, S_, true>)                      \
                                       : go(grp_mma_kernel<bf16_t, CP_, S_, true>);                    \
        return d.dtype == CONV_F16 ? go(grp_mma_kernel<f16_t, CP_, S_, false>)                         \
                                   : go(grp_mma_kernel<bf16_t, CP_, S_, false>);                       \
    }
            MICONV_GM(4, 1) MICONV_GM(8, 1) MICONV_GM(4, 2) MICONV_GM(8, 2)
#undef MICONV_GM
        }
    }
    // Plane schedule: 3x3, equal strides 1 or 2, unit dilation, every
    // group's input and output planes contiguous and 16-byte aligned, one
    // plane per workgroup within the thread and LDS budgets.
    if (two && a.KH == 3 && a.KW == 3 && a.SH == a.SW && (a.SH == 1 || a.SH == 2) && a.DH == 1 && a.DW == 1) {
        const int64_t es = esize(d.dtype);
        constexpr int RB = 2, CB = 7;
        const int64_t S = a.SH;
        const int64_t np = a.npairs;
        const int64_t IHh = (a.OH - 1) * S + 3, IWh = (a.OW - 1) * S + 3;
        const int64_t nrb = cdiv(a.OH, RB), ncb = cdiv(a.OW, CB);
        const int64_t threads = round_up((int64_t)a.Cog * nrb * ncb, 64);
        const int64_t in_words = round_up(np * IHh * IWh, 4);
        const int64_t out_bytes = (int64_t)a.Cog * a.OH * a.OW * es;
        const int64_t lds_total = in_words * 4 + round_up(out_bytes, 16) + 16;   // + a spare slot
        const int64_t in_bytes = (int64_t)a.Cig * a.H * a.W * es;
        const bool xdense = a.xs_w == 1 && a.xs_h == a.W && a.xs_c == (int64_t)a.H * a.W && (a.xs_n * es) % 16 == 0 &&
                            in_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
        const bool ydense = a.ys_w == 1 && a.ys_h == a.OW && a.ys_c == (int64_t)a.OH * a.OW &&
                            (a.ys_n * es) % 16 == 0 && out_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
        if (xdense && ydense && threads <= 512 && cdiv(in_bytes, 16) <= threads && out_bytes / 16 <= 2 * threads &&
            lds_total <= kLds &&
            span(d.x) * es < lim && span(p.y) * es < lim && (int64_t)a.N * a.G < (1LL << 31)) {
            GpLds f;
            f.xs_n = (int32_t)a.xs_n;
            f.ys_n = (int32_t)a.ys_n;
            f.x_bytes = (int32_t)(span(d.x) * es);
            f.y_bytes = (int32_t)(span(p.y) * es);
            f.IHh = (int32_t)IHh;
            f.IWh = (int32_t)IWh;
            f.nrb = (int32_t)nrb;
            f.ncb = (int32_t)ncb;
            f.in_words = (int32_t)in_words;
            f.out_off = (int32_t)(in_words * 4);
            f.chunks_in = (int32_t)cdiv(in_bytes, 16);
            f.pieces_out = (int32_t)(out_bytes / 8);
            int dev = 0, cus = 256;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                cus = 256;
            const dim3 lblock((unsigned)threads);
            const size_t llds = (size_t)lds_total;
            // One resident round of workgroups, spread over the groups.
            auto go = [&](auto kern) {
                int per_cu = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, (int)threads, llds) != hipSuccess ||
                    per_cu < 1)
                    per_cu = 1;
                const int64_t most = std::max<int64_t>(1, std::min<int64_t>(a.N, (int64_t)per_cu * cus / a.G));
                f.wpg = (int32_t)cdiv(a.N, cdiv(a.N, most));
                hipLaunchKernelGGL(kern, dim3((unsigned)((int64_t)a.G * f.wpg)), lblock, llds, s, a, f);
                return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
            };
#define MICONV_GL(NP_, S_)                                                                                      \
    if (np == NP_ && S == S_)                                                                                   \
        return d.dtype == CONV_F16 ? go(grp_lds_kernel<f16_t, NP_, S_, RB, CB>)                                \
                                   : go(grp_lds_kernel<bf16_t, NP_, S_, RB, CB>);
            MICONV_GL(1, 1) MICONV_GL(2, 1) MICONV_GL(3, 1) MICONV_GL(4, 1)
            MICONV_GL(1, 2) MICONV_GL(2, 2) MICONV_GL(3, 2) MICONV_GL(4, 2)
#undef MICONV_GL
        }
    }
    // Flat schedule: a compiled kernel extent (3x3 with equal strides, or one
    // row of 1, 3, 5 or 7 taps; larger square windows exceed the registers),
    // stride 1 or 2, unit dilation, non-negative strides, 32-bit
    // offsets (from the lowered base) and the weights within the LDS budget.
    {
        const bool row1 = a.KH == 1;
        const bool kw_ok = a.KW == 1 || a.KW == 3 || a.KW == 5 || a.KW == 7;
        const int S = a.SW;
        const int R = row1 ? 1 : 4;
        const int64_t nblk = cdiv(a.Cog, 8);
        const int64_t lds_w = nblk * 8 * a.npairs * a.KH * a.KW * 4;
        const int64_t lead = ((int64_t)a.PH * a.xs_h + (int64_t)a.PW * a.xs_w) * esize(d.dtype);
        bool nonneg = true;
        for (int i = 0; i < d.x.rank; ++i) nonneg = nonneg && d.x.strides[i] >= 0;
        for (int i = 0; i < p.y.rank; ++i) nonneg = nonneg && p.y.strides[i] >= 0;
        const int64_t strips = cdiv(a.OH, R);
        const int64_t per_group = (int64_t)a.N * strips * a.OW;
        if (kw_ok && (row1 || (a.KH == a.KW && a.SH == a.SW)) && (S == 1 || S == 2) && a.DH == 1 && a.DW == 1 &&
            nonneg && lds_w <= kLds && span(d.x) * esize(d.dtype) + lead < lim &&
            span(p.y) * esize(d.dtype) < lim && per_group < (1LL << 30) && per_group > 0) {
            GpFlat f;
            f.xs_n = (int32_t)a.xs_n;
            f.xs_c = (int32_t)a.xs_c;
            f.xs_h = (int32_t)a.xs_h;
            f.xs_w = (int32_t)a.xs_w;
            f.ys_n = (int32_t)a.ys_n;
            f.ys_c = (int32_t)a.ys_c;
            f.ys_h = (int32_t)a.ys_h;
            f.ys_w = (int32_t)a.ys_w;
            f.x_bytes = (int32_t)(span(d.x) * esize(d.dtype));
            f.y_bytes = (int32_t)(span(p.y) * esize(d.dtype));
            f.strips = (int32_t)strips;
            f.per_group = (int32_t)per_group;
            f.wpg = (int32_t)cdiv(per_group, 256);
            f.nblk = (int32_t)nblk;
            f.x_lead = (int32_t)lead;
            const dim3 fgrid((unsigned)((int64_t)a.G * f.wpg));
            const size_t flds = (size_t)lds_w;
#define MICONV_GF(KH_, KW_, S_, R_)                                                                              \
    if (a.KH == KH_ && a.KW == KW_ && S == S_) {                                                                \
        if (d.dtype == CONV_F16)                                                                                \
            hipLaunchKernelGGL((grp_flat_kernel<f16_t, KH_, KW_, S_, R_>), fgrid, block, flds, s, a, f);        \
        else                                                                                                    \
            hipLaunchKernelGGL((grp_flat_kernel<bf16_t, KH_, KW_, S_, R_>), fgrid, block, flds, s, a, f);       \
        return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;                                        \
    }
            MICONV_GF(3, 3, 1, 4) MICONV_GF(3, 3, 2, 4)
            MICONV_GF(1, 1, 1, 1) MICONV_GF(1, 3, 1, 1) MICONV_GF(1, 5, 1, 1) MICONV_GF(1, 7, 1, 1)
            MICONV_GF(1, 1, 2, 1) MICONV_GF(1, 3, 2, 1) MICONV_GF(1, 5, 2, 1) MICONV_GF(1, 7, 2, 1)
#undef MICONV_GF
        }
    }
    const bool ext = (a.KW == 3 || a.KW == 5 || a.KW == 7) && (a.KH == 1 || a.KH == a.KW);
    const int64_t tiles = (int64_t)a.N * a.tiles_h * a.tiles_w;
    if (ext && a.DH == 1 && a.DW == 1 && span(d.x) * esize(d.dtype) < lim && span(p.y) * esize(d.dtype) < lim &&
        (int64_t)a.npairs * a.IH * a.IW <= 8 * 256 && a.IH < 32768 && a.IW < 32768) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
        GpPers f;
        f.xs_n = (int32_t)a.xs_n;
        f.xs_c = (int32_t)a.xs_c;
        f.xs_h = (int32_t)a.xs_h;
        f.xs_w = (int32_t)a.xs_w;
        f.ys_n = (int32_t)a.ys_n;
        f.ys_c = (int32_t)a.ys_c;
        f.ys_h = (int32_t)a.ys_h;
        f.ys_w = (int32_t)a.ys_w;
        f.x_bytes = (int32_t)(span(d.x) * esize(d.dtype));
        f.y_bytes = (int32_t)(span(p.y) * esize(d.dtype));
        f.m_plane = (uint32_t)(((1ULL << 32) + (uint64_t)a.IH * a.IW - 1) / ((uint64_t)a.IH * a.IW));
        f.m_iw = (uint32_t)(((1ULL << 32) + a.IW - 1) / a.IW);
        // Four workgroups per CU, spread over the groups.
        f.wpg = (int32_t)std::max<int64_t>(1, std::min<int64_t>(tiles, cdiv(4LL * cus, a.G)));
        const dim3 pgrid((unsigned)((int64_t)a.G * f.wpg));
#define MICONV_GP(KH_, KW_)                                                                                      \
    if (a.KH == KH_ && a.KW == KW_) {                                                                           \
        if (d.dtype == CONV_F16)                                                                                \
            hipLaunchKernelGGL((grp_pers_kernel<f16_t, KH_, KW_, kP, kJB>), pgrid, block, lds, s, a, f);        \
        else                                                                                                    \
            hipLaunchKernelGGL((grp_pers_kernel<bf16_t, KH_, KW_, kP, kJB>), pgrid, block, lds, s, a, f);       \
        return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;                                        \
    }
        MICONV_GP(3, 3) MICONV_GP(5, 5) MICONV_GP(7, 7) MICONV_GP(1, 3) MICONV_GP(1, 5) MICONV_GP(1, 7)
#undef MICONV_GP
    }
    if (d.dtype == CONV_F16)
        hipLaunchKernelGGL((grp_kernel<f16_t, kP, kJB>), grid, block, lds, s, a);
    else if (d.dtype == CONV_BF16)
        hipLaunchKernelGGL((grp_kernel<bf16_t, kP, kJB>), grid, block, lds, s, a);
    else
        return CONV_EUNSUPPORTED;
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
