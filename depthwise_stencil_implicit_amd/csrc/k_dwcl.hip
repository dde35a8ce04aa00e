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
// strip of TO consecutive output columns.  Consecutive lanes hold consecutive
// channel words of the same pixel, so every wave load and store is one
// contiguous run.  Workgroups are persistent -- one resident round over all
// CUs -- and each keeps one (strip chunk, channel chunk), so its weights are
// staged in LDS once; each workgroup walks a contiguous block of output rows.
//
// Rows are streamed once: input row i of a segment feeds the ceil(K/S) output
// rows whose windows cover it, each held in a rolling accumulator slot until
// its last kernel row, where it is stored (rounded once) and the slot reset
// to the bias.  fp16/bf16 take a kernel row as K/2 packed column pairs
// (v_dot2_f32_{f16,bf16}: two products per instruction, fp32 accumulation)
// plus the odd last column as an fp32 FMA; fp32 uses one FMA per tap.
//
// Each wave streams its rows through its own ring of D rows in LDS, filled by
// direct-to-LDS buffer loads (buffer_load_dword ... lds) D-1 rows ahead, so
// D-1 rows of loads are in flight without holding registers.  Loads are raw
// buffer loads: column offsets are computed once, the row offset rides in the
// scalar offset, and absent rows or columns get an out-of-range offset that
// the hardware answers with zeros -- no branch for the padding.  Stores are
// raw buffer stores issued by every step that completes an output row (to an
// out-of-range offset, which the hardware drops, when the row or column is
// absent), so the number of VMEM instructions issued after each ring row is a
// compile-time constant and the wait before reading it is exact.
#include "dev_common.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace miconv {

struct DwArgs {
    const void *x, *w, *b;
    void *y;
    int32_t ys_n, ys_h, ys_w;         // element strides of y (channel stride 1), 32-bit
    int32_t xs_n, xs_h, xs_w;         // element strides of x (channel stride 1), 32-bit
    int32_t x_bytes, y_bytes;         // bytes addressable from x and y (buffer ranges)
    int64_t ws0, ws2, ws3;            // weight strides (output channel, kh, kw)
    int32_t N, H, W, C, OH, OW, pb_h, pb_w;
    int32_t cpb, spb;                 // lane words / strips per workgroup
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

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 in order (a loop whose
// index is a compile-time constant in the body).
template <int... I, class F> __device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(std::make_integer_sequence<int, N>{}, static_cast<F &&>(f));
}

// Stores issued by stream step v: NS when its row completes an output row.
template <int K, int S, int NS> __device__ constexpr int dw_stores_at(int v)
{
    return (((v - (K - 1)) % S) + S) % S == 0 ? NS : 0;
}
// VMEM instructions that may still be pending when step u (position in the
// unrolled block) reads its ring row: the loads (LPR per row) of the D-1 rows
// after it and the stores of the D-1 steps before it -- of this segment only
// when the block is the segment's first (earlier rows came from the prologue).
template <int K, int S, int LPR, int NS, int D> __device__ constexpr int dw_pending_at(int u, bool first)
{
    int n = (D - 1) * LPR;
    for (int d = 1; d < D; ++d)
        if (!first || u - d >= 0) n += dw_stores_at<K, S, NS>(u - d);
    return n;
}
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Weight words per kernel row: 16-bit types keep K/2 packed column pairs
// (kw = 2p, 2p+1) and the last, odd column as fp32; fp32 keeps K fp32 taps.
template <typename T, int K> struct DwTaps {
    static constexpr bool DOT = Word<T>::V == 2;
    static constexpr int KP = DOT ? K / 2 : 0;
    static constexpr int WPR = DOT ? KP + 1 : K;
};

template <typename T, int K, int S, int TO, bool Q>
__global__ __launch_bounds__(256) void dwcl_kernel(DwArgs a)
{
    // The body takes LDS address-space pointers, which only the device pass
    // instantiates; the host pass needs nothing but the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int V = Word<T>::V;
    constexpr int ES = Dt<T>::size;
    constexpr int NCOL = dwcl_ncol(K, S, TO);
    constexpr int INVALID = 0x7fffff00;
    constexpr int M = (K + S - 1) / S;   // output rows open at once (accumulator slots)
    constexpr int U = M * S;             // input rows per unrolled block: slot pattern repeats
    constexpr int D = dwcl_ring_depth(K, S, TO, Q);
    constexpr int LPR = dwcl_loads_per_row(K, S, TO, Q);  // load instructions per input row
    constexpr int NS = dwcl_stores_per_row(TO, Q);        // store instructions per output row
    constexpr int RCOL = dwcl_ring_cols(K, S, TO, Q);     // ring columns per row (>= NCOL)
    constexpr int RING = D * RCOL * 64;  // ring words per wave
    constexpr bool DOT = DwTaps<T, K>::DOT;
    constexpr int KP = DwTaps<T, K>::KP;
    constexpr int WPR = DwTaps<T, K>::WPR;
    static_assert(!DOT || (K & 1), "pairs leave one odd column");
    static_assert(dwcl_pending(K, S, TO, D, Q) <= 63, "vmcnt range");
    // One LDS object: four waves' input-row rings, then (16-byte path) their
    // TO x 64-word output staging tiles.  A single object keeps the compiler's
    // direct-to-LDS tracking from draining the ring around unrelated LDS use.
    __shared__ __attribute__((aligned(16))) uint32_t ring[4 * RING + (Q ? 4 * TO * 64 : 0)];
    uint32_t *stg = ring + 4 * RING;
    typedef __attribute__((address_space(3))) void *lds_ptr;

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

    const int c_base = chc * a.cpb * V;

    // Every wave runs on its own: no barriers.
    const int cl0 = (tid % a.cpb) * V;
    const int c0 = c_base + cl0;
    const int strip = stc * a.spb + tid / a.cpb;
    if (c0 >= a.C || strip >= a.nstrips || tid >= a.cpb * a.spb || first >= last) return;
    const int ow0 = strip * TO;
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t *ringw = ring + wave * RING;        // this wave's ring: [D][RCOL][64 lanes]
    uint32_t *stgw = stg + (Q ? wave * TO * 64 : 0);
    // LDS byte addresses of the staging tile: this lane's word column, and the tile base.
    const uint32_t sa_r = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t *)stgw;
    const uint32_t sa_w = sa_r + 4 * lane;
    const uint32_t *ringl = ringw + lane;

    float bias[V];
    {
        const T *Bp = static_cast<const T *>(a.b);
#pragma unroll
        for (int v = 0; v < V; ++v) bias[v] = a.has_bias ? to_f32(Bp[c0 + v]) : 0.f;
    }

    // This lane's weights, held in registers for the whole walk.  16-bit: per
    // kernel row KP packed column pairs of the stored values per channel
    // (wpl / wph for the low / high channel of the word) and the odd last
    // column as fp32 (wsl / wsh); fp32: every tap (wf).
    uint32_t wpl[K][KP > 0 ? KP : 1], wph[K][KP > 0 ? KP : 1];
    float wsl[K], wsh[K], wf[K][DOT ? 1 : K];
    {
        const T *Wt = static_cast<const T *>(a.w);
        const T *w0 = Wt + (int64_t)c0 * a.ws0;
        const T *w1 = Wt + (int64_t)(V == 2 ? c0 + 1 : c0) * a.ws0;
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            if constexpr (DOT) {
#pragma unroll
                for (int pp = 0; pp < KP; ++pp) {
                    const int64_t o0 = kh * a.ws2 + (2 * pp) * a.ws3, o1 = o0 + a.ws3;
                    wpl[kh][pp] = (uint32_t)w0[o0].u | ((uint32_t)w0[o1].u << 16);
                    wph[kh][pp] = (uint32_t)w1[o0].u | ((uint32_t)w1[o1].u << 16);
                }
                wsl[kh] = to_f32(w0[kh * a.ws2 + (K - 1) * a.ws3]);
                wsh[kh] = to_f32(w1[kh * a.ws2 + (K - 1) * a.ws3]);
            } else {
#pragma unroll
                for (int kw = 0; kw < K; ++kw) wf[kh][kw] = to_f32(w0[kh * a.ws2 + kw * a.ws3]);
            }
        }
    }

    // Column byte offsets of this lane's strip (input and output); absent
    // columns are out of range.  16-byte path: load m of a row brings columns
    // 4m .. 4m+3 of the wave's 64-word run, lane l fetching the 16 bytes of
    // column 4m + l/16, words 4*(l%16) .. +3 -- exactly the [column][lane]
    // order the ring keeps; store s writes chunk 64s + l of the wave's
    // [TO][16 chunks] output tile.
    const int iw0 = ow0 * S - a.pb_w;
    const int cw = c0 - (Q ? lane * V : 0);      // first channel of the wave's run (16-byte path)
    int vcol[LPR], ycol[Q ? 1 : TO];
    if constexpr (Q) {
#pragma unroll
        for (int m = 0; m < LPR; ++m) {
            const int col = 4 * m + (lane >> 4);
            const int iw = iw0 + col;
            vcol[m] = col < NCOL && (unsigned)iw < (unsigned)a.W ? (iw * a.xs_w + cw + 4 * V * (lane & 15)) * ES
                                                                 : INVALID;
        }
    } else {
#pragma unroll
        for (int col = 0; col < NCOL; ++col) {
            const int iw = iw0 + col;
            vcol[col] = (unsigned)iw < (unsigned)a.W ? (iw * a.xs_w + c0) * ES : INVALID;
        }
#pragma unroll
        for (int t = 0; t < TO; ++t) ycol[t] = ow0 + t < a.OW ? ((ow0 + t) * a.ys_w + c0) * ES : INVALID;
    }
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, a.y_bytes, 0x00020000);

    // The block of output rows splits into per-image segments.  In a segment
    // with output rows oh0 + j (j < nj), input row ih0 + i (ih0 = oh0*S - pb)
    // feeds output j at kernel row kh = i - j*S.  Output j lives in
    // accumulator slot j mod M from its first input row to its last; unrolling
    // the stream by U = M*S rows makes every (slot, kh) pair a compile-time
    // constant.
    for (int row0 = first; row0 < last;) {
        const int n = row0 / a.OH;
        const int oh0 = row0 - n * a.OH;
        const int nj = min(last - row0, a.OH - oh0);
        row0 += nj;
        const int ih0 = oh0 * S - a.pb_h;
        const int ni = (nj - 1) * S + K;   // input rows of the segment
        const int xbase = n * a.xs_n;
        const int ybase = n * a.ys_n;

        float acc[M][TO][V];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int t = 0; t < TO; ++t)
#pragma unroll
                for (int v = 0; v < V; ++v) acc[m][t][v] = bias[v];

        // Load input row i into ring slot i mod D (rows past the segment or
        // the image read zeros; they are issued anyway to keep counts fixed).
        auto issue = [&](int i) {
            const int ih = ih0 + i;
            const bool ok = (unsigned)ih < (unsigned)a.H && i < ni;
            const int soff = ok ? (xbase + ih * a.xs_h) * ES : 0;
            const int vbad = ok ? 0 : INVALID;
            uint32_t *dst = ringw + (i % D) * (RCOL * 64);
#pragma unroll
            for (int m = 0; m < LPR; ++m)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(dst + m * (Q ? 256 : 64)), Q ? 16 : 4,
                                                         vcol[m] + vbad, soff, 0, 0);
        };
#pragma unroll
        for (int i = 0; i < D - 1; ++i) issue(i);

        for (int ib = 0; ib < ni; ib += U) {
            static_for<U>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                const int i = ib + u;
                if (i < ni) {
                    issue(i + D - 1);
                    // Wait until row i has landed in the ring.
                    if (ib == 0) wait_vmcnt<dw_pending_at<K, S, LPR, NS, D>(u, true)>();
                    else wait_vmcnt<dw_pending_at<K, S, LPR, NS, D>(u, false)>();
                    asm volatile("" ::: "memory");
                    uint32_t cur[NCOL];
                    const uint32_t *src = ringl + (i % D) * (RCOL * 64);
#pragma unroll
                    for (int col = 0; col < NCOL; ++col) cur[col] = src[col * 64];

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
                    // Open outputs j = ib/S + jp (ib is a multiple of U = M*S) with
                    // kh = u - jp*S in [0, K).
#pragma unroll
                    for (int jp = -M; jp <= M; ++jp) {
                        const int kh = u - jp * S;
                        if (kh < 0 || kh >= K) continue;
                        const int j = ib / S + jp;
                        const int slot = ((jp % M) + M) % M;
                        // Rows outside the segment cost no arithmetic (a uniform
                        // branch); a skipped slot still holds the bias when its
                        // next output (j + M, whose first input row follows j's
                        // last) opens it.
                        if (j >= 0 && j < nj) {
                            if constexpr (DOT) {
#pragma unroll
                                for (int t = 0; t < TO; ++t) {
#pragma unroll
                                    for (int pp = 0; pp < KP; ++pp) {
                                        acc[slot][t][0] = dot2<T>(plo[t * S + 2 * pp], wpl[kh][pp], acc[slot][t][0]);
                                        acc[slot][t][1] = dot2<T>(phi[t * S + 2 * pp], wph[kh][pp], acc[slot][t][1]);
                                    }
                                    acc[slot][t][0] = __builtin_fmaf(xv[t * S + K - 1][0], wsl[kh], acc[slot][t][0]);
                                    acc[slot][t][V - 1] =
                                        __builtin_fmaf(xv[t * S + K - 1][V - 1], wsh[kh], acc[slot][t][V - 1]);
                                }
                            } else {
#pragma unroll
                                for (int t = 0; t < TO; ++t)
#pragma unroll
                                    for (int kw = 0; kw < K; ++kw)
                                        acc[slot][t][0] = __builtin_fmaf(xv[t * S + kw][0], wf[kh][kw], acc[slot][t][0]);
                            }
                        }
                        if (kh == K - 1) {
                            // Output j is complete: NS stores, always issued (dropped
                            // out of range for an absent row or column).
                            const bool ok = j >= 0 && j < nj;
                            const int soff = ok ? (ybase + (oh0 + j) * a.ys_h) * ES : 0;
                            const int vbad = ok ? 0 : INVALID;
                            if constexpr (Q) {
                                // Transpose through the wave's staging tile: word t of
                                // lane l goes to [t][l]; 16-byte chunk k (= 16 t + qd)
                                // then holds words 4 qd .. 4 qd + 3 of column t.  The
                                // staging accesses are LDS instructions with their own
                                // wait, invisible to the compiler's direct-to-LDS wait
                                // logic.
#pragma unroll
                                for (int t = 0; t < TO; ++t) {
                                    const uint32_t wv = Word<T>::narrow(acc[slot][t]);
                                    asm volatile("ds_write_b32 %0, %1" ::"v"(sa_w + t * 256), "v"(wv) : "memory");
                                }
#pragma unroll
                                for (int st = 0; st < NS; ++st) {
                                    const int k = st * 64 + lane, t = k >> 4, qd = k & 15;
                                    const bool in = t < TO && ow0 + t < a.OW;
                                    const uint32_t ra = sa_r + 16 * min(k, 16 * TO - 1);
                                    u32x4 v;
                                    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(ra) : "memory");
                                    const int voff = in ? ((ow0 + t) * a.ys_w + cw + 4 * V * qd) * ES : INVALID;
                                    __builtin_amdgcn_raw_buffer_store_b128(v, yr, voff + vbad, soff, 0);
                                }
                            } else {
#pragma unroll
                                for (int t = 0; t < TO; ++t)
                                    __builtin_amdgcn_raw_buffer_store_b32(Word<T>::narrow(acc[slot][t]), yr,
                                                                          ycol[t] + vbad, soff, 0);
                            }
#pragma unroll
                            for (int t = 0; t < TO; ++t)
#pragma unroll
                                for (int v = 0; v < V; ++v) acc[slot][t][v] = bias[v];
                        }
                    }
                }
            });
        }
    }
#endif
}

namespace {

template <typename T, int K, int S, int TO, bool Q>
hipError_t go(DwArgs a, hipStream_t s)
{
    auto kern = dwcl_kernel<T, K, S, TO, Q>;
    const size_t lds = 0;  // the input-row rings are static LDS
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
hipError_t dispatch(const DwArgs &a, int k, int s, int to, bool q, hipStream_t st)
{
#define MICONV_DW(KK, SS, TT) \
    if (k == KK && s == SS && to == TT) return q ? go<T, KK, SS, TT, true>(a, st) : go<T, KK, SS, TT, false>(a, st);
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
    a.y_bytes = (int32_t)p.tile[3];
    a.ys_n = (int32_t)p.y.strides[0];
    a.ys_h = (int32_t)p.y.strides[2];
    a.ys_w = (int32_t)p.y.strides[3];
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
    a.ch_chunks = (int32_t)p.tile[4];
    a.strip_chunks = (int32_t)p.tile[5];
    a.row_chunks = (int32_t)p.tile[6];
    a.nstrips = (int32_t)cdiv(d.out[1], p.tile[0]);
    a.total = (int32_t)p.grid[0];
    a.has_bias = d.has_bias;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const int k = (int)d.k[0], st = (int)d.stride[0], to = (int)p.tile[0];
    const bool q = p.variant == 1;
    switch (d.dtype) {
    case CONV_F32: e = dispatch<float>(a, k, st, to, q, s); break;
    case CONV_F16: e = dispatch<f16_t>(a, k, st, to, q, s); break;
    default: e = dispatch<bf16_t>(a, k, st, to, q, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
