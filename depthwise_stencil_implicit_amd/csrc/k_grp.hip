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

namespace {
constexpr int kP = 4;
constexpr int kJB = 8;
constexpr int64_t kLds = 64 * 1024;
}  // namespace

bool grp_supported(const conv_desc &d)
{
    if (d.dtype == CONV_F32 || d.transposed) return false;
    if (d.spatial != 1 && d.spatial != 2) return false;
    const int64_t cig = d.C_in / d.groups;
    return cig >= 1 && cig <= 8;
}

void grp_geometry(const conv_desc &d, conv_plan_t &p)
{
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
    p.variant = (int32_t)cog_pad;
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
    a.cog_pad = p.variant;
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
