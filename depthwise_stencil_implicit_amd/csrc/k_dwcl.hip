// Depthwise 2-D stencil for channel-contiguous (channels-last) inputs
// (kernel CONV_K_DW_CL).
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: a direct
// stencil for depthwise convolutions with dilation 1 and kernels up to 9x9,
// with a register sliding-window schedule for channel-contiguous inputs.
//
// Layout on gfx950: x is [N][H][W][C] in memory (C fastest).  A workgroup of
// 256 threads owns CW consecutive 32-bit channel words (two 16-bit channels or
// one fp32 channel each), OCOLS consecutive output columns and one block of
// output rows of one image; thread t computes channel word t % CW for the
// strip of TO output columns t / CW.
//
// Input rows are shared by the workgroup: row i of the block's stream lands
// in slot i mod D of an LDS ring that holds the row's full input span (halo
// columns included) for the workgroup's channel words.  The ring is filled by
// direct-to-LDS buffer loads (buffer_load ... lds) D-1 rows ahead, without
// holding registers; the row offset rides in the scalar offset, and absent
// rows or columns get an out-of-range offset that the hardware answers with
// zeros -- no branch for the padding.  One barrier per row: each wave first
// waits for its own loads of the row, so after the barrier the whole row has
// landed and every wave is done with the previous row, whose slot is then
// refilled.
//
// Rows are streamed once: input row i of a block feeds the ceil(K/S) output
// rows whose windows cover it, each held in a rolling accumulator slot until
// its last kernel row, where it is rounded once, written to an LDS staging
// tile and the slot reset to the bias.  The next step (after its barrier)
// writes the staged row to y with CB-byte stores.  fp16/bf16 multiply packed
// column pairs of one channel with v_dot2_f32_{f16,bf16} (two products per
// instruction, fp32 accumulation); an odd kernel's last column pairs with a
// zero half.  fp32 uses one FMA per tap.  Stores are issued by every step that
// follows a finished output row (dropped out of range for an absent row or
// column).  The wait before reading a ring row allows only the younger ring
// loads to be pending, so the stores issued since are waited for too.
//
// Row blocks of one image alternate direction: odd blocks stream their rows
// bottom to top (the same recurrence with the kernel flipped vertically), so
// two neighbouring blocks, which run side by side on one XCD, read the K-1
// input rows they share at the same time and the second read hits L2.
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
    int32_t ch_chunks, col_chunks;    // workgroup chunks along channel words / output columns
    int32_t rblocks, rpb;             // row blocks per image, output rows per block
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
    __device__ static uint32_t narrow(const float (&f)[2]) { return pack2<bf16_t>(f[0], f[1]); }
};
template <> struct Word<f16_t> {
    static constexpr int V = 2;
    __device__ static uint32_t narrow(const float (&f)[2]) { return pack2<f16_t>(f[0], f[1]); }
};
template <> struct Word<float> {
    static constexpr int V = 1;
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

// Stream step v finishes an output row when its row is the last kernel row of
// some output: v = j*S + K - 1.  The step after it stores that row.
template <int K, int S> __device__ constexpr bool dw_finishes(int v)
{
    return (((v - (K - 1)) % S) + S) % S == 0;
}
template <int K, int S> __device__ constexpr bool dw_stores(int v, bool first)
{
    return (!first || v >= 1) && dw_finishes<K, S>(v - 1);
}
// VMEM instructions that may still be pending when step u (position in the
// unrolled block) waits for its ring row: only the loads (LPW per row) of the
// D-2 rows issued after it.  Loads retire in order among themselves, so a
// count at or below that bound means the row's own loads have landed.  The
// output stores issued in between are not counted: they may retire before
// older loads (measured: with input written by the kernel just before, a
// bound that also allowed the pending stores let a step read a ring row that
// had not landed yet), so they are waited for as well.
template <int K, int S, int LPW, int NS, int D> __device__ constexpr int dw_pending_at(int, bool)
{
    return (D - 2) * LPW;
}
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier for LDS: the wave's own LDS writes complete
// (lgkmcnt(0)) before it arrives, so after the barrier every wave sees every
// wave's writes; unlike __syncthreads() it leaves the ring loads in flight
// (the direct-to-LDS rows are covered by the vmcnt wait before it).
__device__ __forceinline__ void wg_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Packed 16-bit column pairs of one channel, built with one byte permute:
// lo(a, b) = (a.lo, b.lo) and hi(a, b) = (a.hi, b.hi) for channel words a, b
// of two neighbouring columns.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <typename T, int K, int S, int CB>
__global__ __launch_bounds__(256) void dwcl_kernel(DwArgs a)
{
    // The body takes LDS address-space pointers, which only the device pass
    // instantiates; the host pass needs nothing but the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int V = Word<T>::V;
    constexpr int ES = Dt<T>::size;
    constexpr int TO = DW_TO;
    constexpr int CW = dw_cw(S);
    constexpr int OCOLS = dw_ocols(S);
    constexpr int ICOLS = dw_icols(K, S);
    constexpr int WPC = CW * 4 / CB;                 // lanes per column, loads and stores
    constexpr int LPW = dw_lpw(K, S, CB);            // load instructions per wave per row
    constexpr int NS = dw_ns(S, CB);                 // store instructions per thread per output row
    constexpr int ROWB = dw_row_bytes(K, S, CB);     // bytes per ring slot
    constexpr int STGB = dw_stage_bytes(S);          // bytes per staging buffer
    constexpr int D = dw_depth(K, S, CB);
    constexpr int NCOL = (TO - 1) * S + K;           // input columns a lane reads per row
    constexpr int M = (K + S - 1) / S;               // output rows open at once (accumulator slots)
    constexpr int U = M * S;                         // input rows per unrolled block: slot pattern repeats
    constexpr bool DOT = V == 2;
    constexpr int KP = DOT ? (K + 1) / 2 : 1;        // column pairs per kernel row (16-bit)
    constexpr int KK = K * K;
    constexpr int INVALID = 0x7fffff00;
    static_assert(dw_pending(K, S, CB, D) <= 63, "vmcnt range");
    static_assert(CB == 4 || CB == 16, "access width");
    static_assert(CW * V * KK * ES <= dw_tail_bytes(K, S), "weights fit after the ring");
    // One LDS object: the ring, then the two staging buffers (which first
    // hold the workgroup's weights).
    __shared__ __attribute__((aligned(16))) unsigned char lds[D * ROWB + dw_tail_bytes(K, S)];
    unsigned char *stg = lds + D * ROWB;
    typedef __attribute__((address_space(3))) void *lds_ptr;

    // Task: (image, channel/column chunk, row block), row block fastest, so
    // the blocks of one image run side by side on one XCD.
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int SC = a.col_chunks * a.ch_chunks;
    const int task = xcd_block(blockIdx.x, gridDim.x);
    const int rb = task % a.rblocks;
    const int sc = (task / a.rblocks) % SC;
    const int n = task / (a.rblocks * SC);
    const int chc = sc % a.ch_chunks;
    const int colc = sc / a.ch_chunks;
    const int ohA = rb * a.rpb;
    const int nj = min(a.rpb, a.OH - ohA);
    if (n >= a.N || nj <= 0) return;   // uniform over the workgroup
    const bool rev = rb & 1;           // odd blocks stream bottom to top
    const int ni = (nj - 1) * S + K;   // input rows of the block

    // This thread's channel word and output strip.
    const int wd = tid % CW, st = tid / CW;
    const int c0 = (chc * CW + wd) * V;              // first channel of the word
    const bool cok = c0 < a.C;
    const int ow0 = colc * OCOLS + st * TO;          // first output column of the strip
    const int lcol = st * TO * S;                    // its first ring column

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, a.y_bytes, 0x00020000);
    const u32x4 yq = raw_rsrc(a.y, (uint32_t)a.y_bytes);

    // Load lanes: instruction m of wave w fills bytes [(4m + w) * 64 * CB, +64 * CB)
    // of a ring slot; lane l brings chunk (4m + w) * 64 + l, i.e. CB bytes of
    // ring column chunk / WPC at channel-word offset (chunk % WPC) * CB / 4.
    // Columns outside the image, past the span or past the channels read zeros.
    const int col_base = colc * OCOLS * S - a.pb_w;
    const int chw = chc * CW * V;                    // first channel of the workgroup
    int voff[LPW];
#pragma unroll
    for (int m = 0; m < LPW; ++m) {
        const int qd = (m * 4 + wave) * 64 + lane;
        const int col = qd / WPC, w4 = qd % WPC;
        const int iw = col_base + col;
        const int ch = chw + w4 * (CB / ES);
        const bool ok = col < ICOLS && (unsigned)iw < (unsigned)a.W && ch < a.C;
        voff[m] = ok ? (iw * a.xs_w + ch) * ES : INVALID;
    }
    // Store lanes: store r of thread t writes chunk q = r * 256 + t of a staged
    // row, CB bytes of output column q / WPC at channel-word offset
    // (q % WPC) * CB / 4.
    int yoff[NS], soff_l[NS];
#pragma unroll
    for (int r = 0; r < NS; ++r) {
        const int q = r * 256 + tid;
        const int col = q / WPC, w4 = q % WPC;
        const int ow = colc * OCOLS + col;
        const int ch = chw + w4 * (CB / ES);
        const bool ok = col < OCOLS && ow < a.OW && ch < a.C;
        yoff[r] = ok ? (ow * a.ys_w + ch) * ES : INVALID;
        soff_l[r] = min(q, OCOLS * WPC - 1) * CB;
    }

    // Input row of stream step i, and output row of block-local output j.
    const int ih_first = ohA * S - a.pb_h;
    auto in_row = [&](int i) { return rev ? ih_first + ni - 1 - i : ih_first + i; };
    auto out_row = [&](int j) { return rev ? ohA + nj - 1 - j : ohA + j; };
    const int xbase = n * a.xs_n;
    const int ybase = n * a.ys_n;

    // Load input row i into ring slot i mod D (rows past the block or the
    // image read zeros; they are issued anyway to keep counts fixed).  The
    // loads are non-temporal too: the neighbouring block that shares the
    // halo rows reads them at about the same time (measured 2-5% faster).
    auto issue = [&](int i) {
        const int ih = in_row(i);
        const bool ok = (unsigned)ih < (unsigned)a.H && i < ni;
        const int soff = ok ? (xbase + ih * a.xs_h) * ES : 0;
        const int vbad = ok ? 0 : INVALID;
        unsigned char *dst = lds + (i % D) * ROWB + wave * 64 * CB;
#pragma unroll
        for (int m = 0; m < LPW; ++m)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(dst + m * 256 * CB), CB, voff[m] + vbad, soff, 0,
                                                     kStoreNT);
    };
    // Store staged output row j (block-local) from staging buffer j & 1.
    auto store = [&](int j) {
        const bool ok = j >= 0 && j < nj;
        const int soff = ok ? (ybase + out_row(j) * a.ys_h) * ES : 0;
        const int vbad = ok ? 0 : INVALID;
        const unsigned char *src = stg + (j & 1) * STGB;
        if constexpr (CB == 16) {
            // All staged reads first, then the stores: one LDS round trip
            // instead of one per store (the asm stores are barriers to the
            // compiler's scheduling).
            u32x4 v[NS];
#pragma unroll
            for (int r = 0; r < NS; ++r) v[r] = *reinterpret_cast<const u32x4 *>(src + soff_l[r]);
#pragma unroll
            for (int r = 0; r < NS; ++r) store_b128(v[r], yq, yoff[r] + vbad, soff);
        } else {
#pragma unroll
            for (int r = 0; r < NS; ++r) {
                const uint32_t v = *reinterpret_cast<const uint32_t *>(src + soff_l[r]);
                __builtin_amdgcn_raw_buffer_store_b32(v, yr, yoff[r] + vbad, soff, kStoreNT);
            }
        }
    };

    // Weights: the workgroup's CW*V channels x K*K taps, loaded cooperatively
    // (coalesced when the weight is contiguous) into the staging buffers as
    // stored values, in the order (channel, kh, kw).
    {
        const T *Wt = static_cast<const T *>(a.w);
        constexpr int E = CW * V * KK;
        constexpr int PER = (E + 255) / 256;
        T wv[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = r * 256 + tid;
            const int c = e / KK, t = e % KK;
            const int ch = chw + c;
            const bool ok = e < E && ch < a.C;
            const int64_t off = ok ? (int64_t)ch * a.ws0 + (t / K) * a.ws2 + (t % K) * a.ws3 : 0;
            wv[r] = Wt[off];
            if (!ok) __builtin_memset(&wv[r], 0, sizeof(T));
        }
#pragma unroll
        for (int i = 0; i < D; ++i) issue(i);
        T *ws = reinterpret_cast<T *>(stg);
#pragma unroll
        for (int r = 0; r < PER; ++r)
            if (r * 256 + tid < E) ws[r * 256 + tid] = wv[r];
    }
    wg_barrier();

    float bias[V];
    {
        const T *Bp = static_cast<const T *>(a.b);
        const int cc = cok ? c0 : 0;
#pragma unroll
        for (int v = 0; v < V; ++v) bias[v] = a.has_bias ? to_f32(Bp[cc + v]) : 0.f;
    }
    // This thread's weights, in registers for the whole block.  Kernel row kh
    // of the stream is stored row kh (K-1-kh when streaming bottom to top).
    // 16-bit: per kernel row KP packed column pairs (kw = 2p, 2p+1) of the
    // stored values per channel, an odd kernel's last pair completed with zero
    // (wpl / wph for the low / high channel of the word); fp32: every tap (wf).
    uint32_t wpl[K][KP], wph[K][KP];
    float wf[K][DOT ? 1 : K];
    {
        const uint16_t *w16 = reinterpret_cast<const uint16_t *>(stg);
        const float *w32 = reinterpret_cast<const float *>(stg);
        const int cl = wd * V;   // local channel
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            const int sr = rev ? K - 1 - kh : kh;
            if constexpr (DOT) {
#pragma unroll
                for (int pp = 0; pp < KP; ++pp) {
                    const int t0 = sr * K + 2 * pp;
                    const bool two = 2 * pp + 1 < K;
                    wpl[kh][pp] = (uint32_t)w16[cl * KK + t0] | (two ? (uint32_t)w16[cl * KK + t0 + 1] << 16 : 0u);
                    wph[kh][pp] =
                        (uint32_t)w16[(cl + 1) * KK + t0] | (two ? (uint32_t)w16[(cl + 1) * KK + t0 + 1] << 16 : 0u);
                }
            } else {
#pragma unroll
                for (int kw = 0; kw < K; ++kw) wf[kh][kw] = w32[cl * KK + sr * K + kw];
            }
        }
    }

    float acc[M][TO][V];
    const uint32_t *ringw = reinterpret_cast<const uint32_t *>(lds) + lcol * CW + wd;
    uint32_t *stgw = reinterpret_cast<uint32_t *>(stg) + st * TO * CW + wd;
    auto read_row = [&](int i, uint32_t (&dst)[NCOL]) {
        const uint32_t *src = ringw + (i % D) * (ROWB / 4);
#pragma unroll
        for (int col = 0; col < NCOL; ++col) dst[col] = src[col * CW];
    };
    // Row 0 in registers; from then on step i reads row i+1 while it
    // multiplies row i.
    uint32_t cur[NCOL];
    wait_vmcnt<(D - 1) * LPW>();
    wg_barrier();
    read_row(0, cur);

    // Stream step i (row in_row(i)) feeds block-local output j at kernel row
    // kh = i - j*S.  Output j lives in accumulator slot j mod M from its first
    // input row (kh = 0, which starts from the bias) to its last; unrolling the
    // stream by U = M*S rows makes every (slot, kh) pair a compile-time
    // constant.
    for (int ib = 0; ib < ni; ib += U) {
        static_for<U>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            const int i = ib + u;
            if (i < ni) {
                // Own loads of row i+1 landed; after the barrier every wave's
                // have, every wave holds row i in registers (its slot is
                // refilled next), and the row finished in step i-1 is staged.
                if (ib == 0) wait_vmcnt<dw_pending_at<K, S, LPW, NS, D>(u, true)>();
                else wait_vmcnt<dw_pending_at<K, S, LPW, NS, D>(u, false)>();
                wg_barrier();
                issue(i + D);
                if (ib == 0) {
                    if constexpr (dw_stores<K, S>(u, true)) store((i - 1 - (K - 1)) / S);
                } else {
                    if constexpr (dw_stores<K, S>(u, false)) store((i - 1 - (K - 1)) / S);
                }
                uint32_t nxt[NCOL];
                read_row(i + 1, nxt);

                // Row operands.  16-bit: column pairs (c, c+1) of each channel,
                // and an odd kernel's last column with a zero partner; fp32: the
                // columns as they are.  Entries no tap uses fold away.
                uint32_t plo[NCOL], phi[NCOL], zlo[NCOL], zhi[NCOL];
#pragma unroll
                for (int col = 0; col < NCOL; ++col) {
                    if constexpr (DOT) {
                        if (col + 1 < NCOL) {
                            plo[col] = pair_lo(cur[col], cur[col + 1]);
                            phi[col] = pair_hi(cur[col], cur[col + 1]);
                        }
                        zlo[col] = cur[col] & 0xffffu;
                        zhi[col] = cur[col] >> 16;
                    }
                }
                // Open outputs j = ib/S + jp (ib is a multiple of U = M*S) with
                // kh = u - jp*S in [0, K).
#pragma unroll
                for (int jp = -M; jp <= M; ++jp) {
                    const int kh = u - jp * S;
                    if (kh < 0 || kh >= K) continue;
                    const int j = ib / S + jp;
                    const int slot = ((jp % M) + M) % M;
                    // Rows outside the block cost no arithmetic (a uniform
                    // branch); an output's first kernel row starts from the bias.
                    if (j >= 0 && j < nj) {
#pragma unroll
                        for (int t = 0; t < TO; ++t) {
                            if constexpr (DOT) {
                                float a0 = acc[slot][t][0];
                                float a1 = acc[slot][t][1];
#pragma unroll
                                for (int pp = 0; pp < KP; ++pp) {
                                    const int col = t * S + 2 * pp;
                                    const bool two = 2 * pp + 1 < K;
                                    const uint32_t x0 = two ? plo[col] : zlo[col], x1 = two ? phi[col] : zhi[col];
                                    if (kh == 0 && pp == 0) {
                                        // The output's first product starts from the bias.
                                        a0 = dot2_to<T>(x0, wpl[kh][pp], bias[0]);
                                        a1 = dot2_to<T>(x1, wph[kh][pp], bias[1]);
                                    } else {
                                        a0 = dot2<T>(x0, wpl[kh][pp], a0);
                                        a1 = dot2<T>(x1, wph[kh][pp], a1);
                                    }
                                }
                                acc[slot][t][0] = a0;
                                acc[slot][t][1] = a1;
                            } else {
                                float a0 = kh == 0 ? bias[0] : acc[slot][t][0];
#pragma unroll
                                for (int kw = 0; kw < K; ++kw)
                                    a0 = __builtin_fmaf(__uint_as_float(cur[t * S + kw]), wf[kh][kw], a0);
                                acc[slot][t][0] = a0;
                            }
                        }
                    }
                    if (kh == K - 1) {
                        // Output j is complete: round once into staging buffer
                        // j & 1 (the next step stores it).
                        uint32_t *dst = stgw + (j & 1) * (STGB / 4);
#pragma unroll
                        for (int t = 0; t < TO; ++t) dst[t * CW] = Word<T>::narrow(acc[slot][t]);
                    }
                }
#pragma unroll
                for (int col = 0; col < NCOL; ++col) cur[col] = nxt[col];
            }
        });
    }
    // The last output row was staged by the last step: store it once every
    // wave has written its part.
    wg_barrier();
    store(nj - 1);
#endif
}

namespace {

template <typename T, int K, int S, int CB>
hipError_t go(DwArgs a, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL((dwcl_kernel<T, K, S, CB>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T, int CB>
hipError_t dispatch(const DwArgs &a, int64_t grid, int k, int s, hipStream_t st)
{
#define MICONV_DW(KK, SS) \
    if (k == KK && s == SS) return go<T, KK, SS, CB>(a, grid, st);
    MICONV_DW(3, 1) MICONV_DW(5, 1) MICONV_DW(7, 1) MICONV_DW(3, 2) MICONV_DW(5, 2) MICONV_DW(7, 2)
    MICONV_DW(9, 1) MICONV_DW(9, 2)
#undef MICONV_DW
    return hipErrorInvalidValue;
}

}  // namespace

// ---- generic schedule (plan variant DWCL_GENERIC) ----
//
// Channel-contiguous depthwise calls the ring kernels do not cover -- any
// channel multiplier m (output channel co reads input channel co / m: the
// multiplier schedule of the PR #25085 description), kernels up to 9 x 9 of
// any shape, any stride, 1-D calls lifted to one row -- with no LDS: lane
// (channel word, column strip) of a 256-thread workgroup owns one 32-bit
// word of output channels (two 16-bit or one fp32) and TO consecutive output
// columns of one output row; consecutive lanes take consecutive channel
// words, so every load and store of the workgroup is a run of consecutive
// channels.  Input values come straight from global memory (the K x K window
// re-reads hit L1/L2), one word load for both channels of a word when m = 1,
// one element load when both output channels share an input channel (m
// even), two otherwise.  fp32 accumulation, bias first, one rounding.
struct DwgArgs {
    const void *x, *w, *b;
    void *y;
    int64_t xs_n, xs_h, xs_w;     // element strides of x (channel stride 1)
    int64_t ys_n, ys_h, ys_w;     // element strides of y
    int64_t ys_c;                 // channel stride of y: 1, or positions contiguous (ys_w == 1)
    int64_t ws0, ws2, ws3;        // weight strides (output channel, kh, kw)
    int32_t H, W, M, Cout, OH, OW, KH, KW, SH, SW, PH, PW;
    int32_t col_blocks, ch_blocks, has_bias;
    int32_t x_bytes, w_bytes;     // buffer ranges: x from the image's start, the weights
};

constexpr int DWG_TO = 8;         // output columns per lane

// KB: kernel width rounded up to 3, 5 or 9 (taps past the width have zero
// weights); S: the column stride (1..3).  Per kernel row the lane first loads
// its whole input window -- (TO-1)*S + KB columns, absent ones as zeros --
// and the kernel row's weights, all loads in flight together, then runs the
// TO x KB multiply-adds from registers.
template <typename T, bool WX, int KB, int S>
__global__ __launch_bounds__(256) void dwg_kernel(DwgArgs a)
{
    constexpr int V = Dt<T>::size == 2 ? 2 : 1;
    constexpr int TO = DWG_TO;
    constexpr int NX = (TO - 1) * S + KB;        // input columns of the window
    const int tid = threadIdx.x, cl = tid & 31, st = tid >> 5;
    int b = blockIdx.x;
    const int chb = b % a.ch_blocks;
    b /= a.ch_blocks;
    const int cb = b % a.col_blocks;
    b /= a.col_blocks;
    const int oh = b % a.OH;
    const int n = b / a.OH;
    const int co0 = (chb * 32 + cl) * V;          // first output channel of the lane
    const int ow0 = (cb * 8 + st) * TO;          // first output column of the lane
    if (co0 >= a.Cout || ow0 >= a.OW) return;    // no barriers below
    const int nv = min(V, a.Cout - co0);         // output channels of the word
    int ci[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ci[v] = min(co0 + v, a.Cout - 1) / a.M;
    const bool same = V == 2 && ci[0] == ci[V - 1];

    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    float acc[TO][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const float bv = (a.has_bias && v < nv) ? to_f32(Bp[co0 + v]) : 0.f;
#pragma unroll
        for (int t = 0; t < TO; ++t) acc[t][v] = bv;
    }
    constexpr int ES = (int)sizeof(T);
    constexpr int INVALID = 0x7fffff00;
    const int iw0 = ow0 * S - a.PW;
    const int nx = (min(TO, a.OW - ow0) - 1) * S + a.KW;   // window columns any output uses
    const int ih0 = oh * a.SH - a.PH;
    // Buffer loads from this image of x and from the weights: per-lane byte
    // offsets of the window columns and the weight taps are the same for
    // every kernel row (absent columns get an offset the buffer range
    // drops, which reads zero); the row rides in the scalar offset.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(static_cast<const T *>(a.x) + (int64_t)n * a.xs_n), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.w), (short)0, a.w_bytes, 0x00020000);
    int xo[NX][V], wb[V];
#pragma unroll
    for (int j = 0; j < NX; ++j) {
        const int iw = iw0 + j;
        const bool ok = j < nx && (unsigned)iw < (unsigned)a.W;
        xo[j][0] = ok ? (iw * (int)a.xs_w + (WX ? co0 : ci[0])) * ES : INVALID;
        if constexpr (V == 2) xo[j][1] = ok ? (iw * (int)a.xs_w + ci[1]) * ES : INVALID;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) wb[v] = v < nv ? (co0 + v) * (int)a.ws0 * ES : INVALID;
    // Kernel rows are software-pipelined: the next row's window and weights
    // are loaded (as raw bits, converted only when used) while the current
    // row is multiplied, so each row does not wait out a load latency of its
    // own.  Rows outside the input load nothing and multiply nothing.
    auto val = [](uint32_t u) -> float {
        if constexpr (sizeof(T) == 2) {
            T t;
            t.u = (uint16_t)u;
            return to_f32(t);
        } else {
            return __uint_as_float(u);
        }
    };
    auto ld = [](__amdgpu_buffer_rsrc_t r, int voff, int soff) -> uint32_t {
        if constexpr (sizeof(T) == 2) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
        else return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    };
    auto fetch = [&](int kh, uint32_t (&px)[NX][V], uint32_t (&pw)[KB][V]) {
        const int ih = ih0 + kh;
        if ((unsigned)ih >= (unsigned)a.H) return;   // uniform over the workgroup
        const int xs = ih * (int)a.xs_h * ES, ws = kh * (int)a.ws2 * ES;
#pragma unroll
        for (int kw = 0; kw < KB; ++kw)
#pragma unroll
            for (int v = 0; v < V; ++v) pw[kw][v] = kw < a.KW ? ld(wr, wb[v], ws + kw * (int)a.ws3 * ES) : 0u;
#pragma unroll
        for (int j = 0; j < NX; ++j) {
            if constexpr (WX) {
                // m = 1, 16-bit: the word of input channels co0, co0 + 1.
                px[j][0] = __builtin_amdgcn_raw_buffer_load_b32(xr, xo[j][0], xs, 0);
            } else {
                px[j][0] = ld(xr, xo[j][0], xs);
                if constexpr (V == 2) px[j][1] = same ? px[j][0] : ld(xr, xo[j][1], xs);
            }
        }
    };
    uint32_t rx[NX][V], rw[KB][V];
    fetch(0, rx, rw);
    for (int kh = 0; kh < a.KH; ++kh) {
        uint32_t qx[NX][V], qw[KB][V];
        const bool more = kh + 1 < a.KH;
        if (more) fetch(kh + 1, qx, qw);
        if ((unsigned)(ih0 + kh) < (unsigned)a.H) {
            float wv[KB][V], xw[NX][V];
#pragma unroll
            for (int kw = 0; kw < KB; ++kw)
#pragma unroll
                for (int v = 0; v < V; ++v) wv[kw][v] = val(rw[kw][v]);
#pragma unroll
            for (int j = 0; j < NX; ++j) {
                if constexpr (WX) {
                    xw[j][0] = val(rx[j][0] & 0xffffu);
                    xw[j][V - 1] = val(rx[j][0] >> 16);
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v) xw[j][v] = val(rx[j][v]);
                }
            }
#pragma unroll
            for (int t = 0; t < TO; ++t)
#pragma unroll
                for (int kw = 0; kw < KB; ++kw)
#pragma unroll
                    for (int v = 0; v < V; ++v) acc[t][v] = __builtin_fmaf(xw[t * S + kw][v], wv[kw][v], acc[t][v]);
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < NX; ++j)
#pragma unroll
                for (int v = 0; v < V; ++v) rx[j][v] = qx[j][v];
#pragma unroll
            for (int kw = 0; kw < KB; ++kw)
#pragma unroll
                for (int v = 0; v < V; ++v) rw[kw][v] = qw[kw][v];
        }
    }
    T *__restrict__ Yb = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + (int64_t)oh * a.ys_h;
    if (a.ys_c != 1) {
        // Positions contiguous in y (the channel-major output of a 1-D call on
        // a channels-last input): each output channel's TO results are one
        // run, stored as 16-byte vectors where the run is whole and aligned,
        // else element by element.
        constexpr int NW32 = TO * (int)sizeof(T) / 4;   // 32-bit words of a run
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (v >= nv) break;
            T *py = Yb + (int64_t)(co0 + v) * a.ys_c + ow0;
            if (ow0 + TO <= a.OW && (reinterpret_cast<uintptr_t>(py) & 15) == 0) {
                uint32_t wd[NW32];
#pragma unroll
                for (int q = 0; q < NW32; ++q) {
                    if constexpr (sizeof(T) == 2)
                        wd[q] = pack2<T>(acc[2 * q][v], acc[2 * q + 1][v]);
                    else
                        wd[q] = __float_as_uint(acc[q][v]);
                }
#pragma unroll
                for (int q = 0; q < NW32; q += 4)
                    *reinterpret_cast<uint4 *>(reinterpret_cast<uint32_t *>(py) + q) =
                        uint4{wd[q], wd[q + 1], wd[q + 2], wd[q + 3]};
            } else {
#pragma unroll
                for (int t = 0; t < TO; ++t)
                    if (ow0 + t < a.OW) py[t] = from_f32<T>(acc[t][v]);
            }
        }
        return;
    }
    T *__restrict__ Y = Yb + co0;
#pragma unroll
    for (int t = 0; t < TO; ++t) {
        const int ow = ow0 + t;
        if (ow >= a.OW) break;
        T *py = Y + (int64_t)ow * a.ys_w;
        if constexpr (V == 2) {
            if (nv == 2) {
                *reinterpret_cast<uint32_t *>(py) = pack2<T>(acc[t][0], acc[t][1]);
                continue;
            }
        }
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (v < nv) py[v] = from_f32<T>(acc[t][v]);
    }
}

// The multiplier schedule (16-bit, m = MO in {2, 4}): lane = one word of
// INPUT channels (c0, c0 + 1) x TO output columns; it computes all 2 MO
// output channels c0*m .. c0*m + 2m - 1 of its two input channels from one
// word load per window column (the multiplier fan-out), and stores them as
// one 8- or 16-byte run per output column.
template <typename T, int MO, int KB, int S>
__global__ __launch_bounds__(256) void dwm_kernel(DwgArgs a)
{
    constexpr int TO = DWG_TO;
    constexpr int NX = (TO - 1) * S + KB;
    constexpr int NO = 2 * MO;                   // output channels per lane
    const int tid = threadIdx.x, cl = tid & 31, st = tid >> 5;
    int b = blockIdx.x;
    const int chb = b % a.ch_blocks;
    b /= a.ch_blocks;
    const int cb = b % a.col_blocks;
    b /= a.col_blocks;
    const int oh = b % a.OH;
    const int n = b / a.OH;
    const int Cin = a.Cout / MO;
    const int c0 = (chb * 32 + cl) * 2;          // first input channel of the lane
    const int ow0 = (cb * 8 + st) * TO;
    if (c0 >= Cin || ow0 >= a.OW) return;        // no barriers below
    const int co0 = c0 * MO;
    const bool two = c0 + 1 < Cin;               // both input channels present

    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    float acc[TO][NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) {
        const float bv = (a.has_bias && (o < MO || two)) ? to_f32(Bp[co0 + o]) : 0.f;
#pragma unroll
        for (int t = 0; t < TO; ++t) acc[t][o] = bv;
    }
    constexpr int INVALID = 0x7fffff00;
    const int iw0 = ow0 * S - a.PW;
    const int nx = (min(TO, a.OW - ow0) - 1) * S + a.KW;
    const int ih0 = oh * a.SH - a.PH;
    // Buffer loads with per-lane offsets fixed over the kernel rows and the
    // next row's words and weights in flight while the current row is
    // multiplied (as in the generic kernel above).
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(static_cast<const T *>(a.x) + (int64_t)n * a.xs_n), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.w), (short)0, a.w_bytes, 0x00020000);
    int xo[NX], wb[NO];
#pragma unroll
    for (int j = 0; j < NX; ++j) {
        const int iw = iw0 + j;
        xo[j] = (j < nx && (unsigned)iw < (unsigned)a.W) ? (iw * (int)a.xs_w + c0) * 2 : INVALID;
    }
#pragma unroll
    for (int o = 0; o < NO; ++o) wb[o] = (o < MO || two) ? (co0 + o) * (int)a.ws0 * 2 : INVALID;
    auto fetch = [&](int kh, uint32_t (&px)[NX], uint32_t (&pw)[KB][NO]) {
        const int ih = ih0 + kh;
        if ((unsigned)ih >= (unsigned)a.H) return;   // uniform over the workgroup
        const int xs = ih * (int)a.xs_h * 2, ws = kh * (int)a.ws2 * 2;
#pragma unroll
        for (int kw = 0; kw < KB; ++kw)
#pragma unroll
            for (int o = 0; o < NO; ++o)
                pw[kw][o] =
                    kw < a.KW ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wr, wb[o], ws + kw * (int)a.ws3 * 2, 0) : 0u;
#pragma unroll
        for (int j = 0; j < NX; ++j) px[j] = __builtin_amdgcn_raw_buffer_load_b32(xr, xo[j], xs, 0);
    };
    auto val = [](uint32_t u) -> float {
        T t;
        t.u = (uint16_t)u;
        return to_f32(t);
    };
    uint32_t rx[NX], rw[KB][NO];
    fetch(0, rx, rw);
    for (int kh = 0; kh < a.KH; ++kh) {
        uint32_t qx[NX], qw[KB][NO];
        const bool more = kh + 1 < a.KH;
        if (more) fetch(kh + 1, qx, qw);
        if ((unsigned)(ih0 + kh) < (unsigned)a.H) {
            float wv[KB][NO], xw[NX][2];
#pragma unroll
            for (int kw = 0; kw < KB; ++kw)
#pragma unroll
                for (int o = 0; o < NO; ++o) wv[kw][o] = val(rw[kw][o]);
#pragma unroll
            for (int j = 0; j < NX; ++j) {
                xw[j][0] = val(rx[j] & 0xffffu);
                xw[j][1] = val(rx[j] >> 16);
            }
#pragma unroll
            for (int t = 0; t < TO; ++t)
#pragma unroll
                for (int kw = 0; kw < KB; ++kw)
#pragma unroll
                    for (int o = 0; o < NO; ++o)
                        acc[t][o] = __builtin_fmaf(xw[t * S + kw][o / MO], wv[kw][o], acc[t][o]);
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < NX; ++j) rx[j] = qx[j];
#pragma unroll
            for (int kw = 0; kw < KB; ++kw)
#pragma unroll
                for (int o = 0; o < NO; ++o) rw[kw][o] = qw[kw][o];
        }
    }
    T *__restrict__ Y = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + (int64_t)oh * a.ys_h + co0;
#pragma unroll
    for (int t = 0; t < TO; ++t) {
        const int ow = ow0 + t;
        if (ow >= a.OW) break;
        T *py = Y + (int64_t)ow * a.ys_w;
        uint32_t wd[MO];
#pragma unroll
        for (int q = 0; q < MO; ++q) wd[q] = pack2<T>(acc[t][2 * q], acc[t][2 * q + 1]);
        if (two) {
            if constexpr (MO == 2) {
                *reinterpret_cast<uint2 *>(py) = uint2{wd[0], wd[1]};
            } else {
                *reinterpret_cast<uint4 *>(py) = uint4{wd[0], wd[1], wd[2], wd[3]};
            }
        } else {
#pragma unroll
            for (int q = 0; q < MO / 2; ++q) reinterpret_cast<uint32_t *>(py)[q] = wd[q];
        }
    }
}

namespace {

// Transposed depthwise calls (multiplier 1, dilation 1) on the same lane
// layout: output o reads input (o + pb - t)/s at tap t when the quotient is an
// exact integer inside the input, per dim (executorch PR #25091 description,
// second paragraph).  Lane = one word of channels (two 16-bit or one fp32) x
// DWG_TO consecutive output columns of one output row.  With the column
// stride S (1 or 2) dividing DWG_TO, every lane's first column is a multiple
// of S, so the phase (o + pb) mod S of each of its columns is fixed by the
// launch's PHW = pb mod S: which (column, tap) pairs meet, and at which input
// column of the lane's window, is decided at compile time.  Rows are
// uniform over the workgroup: a kernel row whose numerator is not a multiple
// of the row stride, or that falls outside the input, is skipped.  x is read
// as channel words where it is word-aligned with an even channel count (WX),
// else element by element; element stores at y's strides; fp32 accumulation
// from the bias, one rounding.
__host__ __device__ constexpr int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

template <typename T, int KB, int S, int PHW, bool WX>
__global__ __launch_bounds__(256) void dwt_kernel(DwgArgs a)
{
    constexpr int V = Dt<T>::size == 2 ? 2 : 1;
    constexpr int TO = DWG_TO;
    static_assert(TO % S == 0, "column phase");
    constexpr int JMIN = floor_div(PHW - (KB - 1), S), JMAX = floor_div(TO - 1 + PHW, S);
    constexpr int NX = JMAX - JMIN + 1;          // input columns of the lane's window
    const int tid = threadIdx.x, cl = tid & 31, st = tid >> 5;
    int b = blockIdx.x;
    const int chb = b % a.ch_blocks;
    b /= a.ch_blocks;
    const int cb = b % a.col_blocks;
    b /= a.col_blocks;
    const int oh = b % a.OH;
    const int n = b / a.OH;
    const int co0 = (chb * 32 + cl) * V;
    const int ow0 = (cb * 8 + st) * TO;
    if (co0 >= a.Cout || ow0 >= a.OW) return;
    const int nv = min(V, a.Cout - co0);
    const T *__restrict__ X = static_cast<const T *>(a.x) + (int64_t)n * a.xs_n + co0;
    const T *__restrict__ Wt = static_cast<const T *>(a.w);
    const T *__restrict__ Bp = static_cast<const T *>(a.b);
    float acc[TO][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const float bv = (a.has_bias && v < nv) ? to_f32(Bp[co0 + v]) : 0.f;
#pragma unroll
        for (int t = 0; t < TO; ++t) acc[t][v] = bv;
    }
    const int base = (ow0 + a.PW - PHW) / S + JMIN;   // first input column of the window
    for (int kh = 0; kh < a.KH; ++kh) {
        const int num = oh + a.PH - kh;
        if (num < 0 || num % a.SH) continue;
        const int ih = num / a.SH;
        if (ih >= a.H) continue;
        float wv[KB][V], xw[NX][V];
#pragma unroll
        for (int kw = 0; kw < KB; ++kw)
#pragma unroll
            for (int v = 0; v < V; ++v)
                wv[kw][v] = (kw < a.KW && v < nv)
                                ? to_f32(Wt[(int64_t)(co0 + v) * a.ws0 + (int64_t)kh * a.ws2 + (int64_t)kw * a.ws3])
                                : 0.f;
        const T *xr = X + (int64_t)ih * a.xs_h;
#pragma unroll
        for (int j = 0; j < NX; ++j) {
            const int iw = base + j;
            const bool ok = (unsigned)iw < (unsigned)a.W;
            if constexpr (WX) {
                // Both channels of the word in one 4-byte load (even C,
                // word-aligned x).
                const uint32_t u = ok ? *reinterpret_cast<const uint32_t *>(xr + (int64_t)iw * a.xs_w) : 0u;
                xw[j][0] = lo_f32(u, T{});
                xw[j][V - 1] = hi_f32(u, T{});
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) xw[j][v] = (ok && v < nv) ? to_f32(xr[(int64_t)iw * a.xs_w + v]) : 0.f;
            }
        }
#pragma unroll
        for (int t = 0; t < TO; ++t)
#pragma unroll
            for (int kw = 0; kw < KB; ++kw) {
                if (((t + PHW - kw) % S + S) % S != 0) continue;
                const int j = floor_div(t + PHW - kw, S) - JMIN;
#pragma unroll
                for (int v = 0; v < V; ++v) acc[t][v] = __builtin_fmaf(xw[j][v], wv[kw][v], acc[t][v]);
            }
    }
    T *__restrict__ Y = static_cast<T *>(a.y) + (int64_t)n * a.ys_n + (int64_t)oh * a.ys_h + (int64_t)co0 * a.ys_c;
#pragma unroll
    for (int t = 0; t < TO; ++t) {
        const int ow = ow0 + t;
        if (ow >= a.OW) break;
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (v < nv) Y[(int64_t)ow * a.ys_w + (int64_t)v * a.ys_c] = from_f32<T>(acc[t][v]);
    }
}

template <typename T, bool WX>
hipError_t dwt_go(const DwgArgs &a, dim3 grid, hipStream_t s)
{
    const int kb = a.KW <= 3 ? 3 : (a.KW <= 5 ? 5 : (a.KW <= 7 ? 7 : 9));
    const int ph = a.PW % a.SW;
#define MICONV_DWT(KB_, S_, P_) \
    if (kb == KB_ && a.SW == S_ && ph == P_) hipLaunchKernelGGL((dwt_kernel<T, KB_, S_, P_, WX>), grid, dim3(256), 0, s, a); else
    MICONV_DWT(3, 1, 0) MICONV_DWT(5, 1, 0) MICONV_DWT(7, 1, 0) MICONV_DWT(9, 1, 0)
    MICONV_DWT(3, 2, 0) MICONV_DWT(5, 2, 0) MICONV_DWT(7, 2, 0) MICONV_DWT(9, 2, 0)
    MICONV_DWT(3, 2, 1) MICONV_DWT(5, 2, 1) MICONV_DWT(7, 2, 1) MICONV_DWT(9, 2, 1) return hipErrorInvalidValue;
#undef MICONV_DWT
    return hipGetLastError();
}

template <typename T, bool WX>
hipError_t dwg_go(const DwgArgs &a, dim3 grid, hipStream_t s)
{
    const int kb = a.KW <= 3 ? 3 : (a.KW <= 5 ? 5 : 9);
#define MICONV_DWG(KB_, S_) \
    if (kb == KB_ && a.SW == S_) hipLaunchKernelGGL((dwg_kernel<T, WX, KB_, S_>), grid, dim3(256), 0, s, a); else
    MICONV_DWG(3, 1) MICONV_DWG(5, 1) MICONV_DWG(9, 1) MICONV_DWG(3, 2) MICONV_DWG(5, 2) MICONV_DWG(9, 2)
    MICONV_DWG(3, 3) MICONV_DWG(5, 3) MICONV_DWG(9, 3) return hipErrorInvalidValue;
#undef MICONV_DWG
    return hipGetLastError();
}

}  // namespace

int launch_dwg(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream)
{
    const conv_desc &d = p.d;
    const bool two = d.spatial == 2;
    DwgArgs a;
    a.x = x;
    a.w = w;
    a.b = b;
    a.y = y;
    a.xs_n = d.x.strides[0];
    a.xs_h = two ? d.x.strides[2] : 0;
    a.xs_w = d.x.strides[two ? 3 : 2];
    a.ys_n = p.y.strides[0];
    a.ys_h = two ? p.y.strides[2] : 0;
    a.ys_w = p.y.strides[two ? 3 : 2];
    a.ys_c = p.y.strides[1];
    a.ws0 = d.w.strides[0];
    a.ws2 = two ? d.w.strides[2] : 0;
    a.ws3 = d.w.strides[two ? 3 : 2];
    a.H = two ? (int32_t)d.in[0] : 1;
    a.W = (int32_t)d.in[two ? 1 : 0];
    a.M = (int32_t)(d.C_out / d.C_in);
    a.Cout = (int32_t)d.C_out;
    a.OH = two ? (int32_t)d.out[0] : 1;
    a.OW = (int32_t)d.out[two ? 1 : 0];
    a.KH = two ? (int32_t)d.k[0] : 1;
    a.KW = (int32_t)d.k[two ? 1 : 0];
    a.SH = two ? (int32_t)d.stride[0] : 1;
    a.SW = (int32_t)d.stride[two ? 1 : 0];
    a.PH = two ? (int32_t)d.padding_before[0] : 0;
    a.PW = (int32_t)d.padding_before[two ? 1 : 0];
    a.col_blocks = (int32_t)p.tile[DW_COLCHUNKS];
    a.ch_blocks = (int32_t)p.tile[DW_CHCHUNKS];
    a.has_bias = d.has_bias;
    {
        // One image of x (every dim but the batch) and the weight, in bytes;
        // the planner keeps both below 2^31.
        const int64_t es = esize(d.dtype);
        int64_t xi = 0, wi = 0;
        for (int i = 1; i < d.x.rank; ++i) xi += (d.x.sizes[i] - 1) * d.x.strides[i];
        for (int i = 0; i < d.w.rank; ++i) wi += (d.w.sizes[i] - 1) * d.w.strides[i];
        a.x_bytes = (int32_t)((xi + 1) * es);
        a.w_bytes = (int32_t)((wi + 1) * es);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)p.grid[0]);
    if (d.transposed) {
        // Word loads of x: 16-bit, even channel count, x word-aligned.
        const bool twx = esize(d.dtype) == 2 && d.C_in % 2 == 0 && (reinterpret_cast<uintptr_t>(x) & 3) == 0 &&
                         a.xs_n % 2 == 0 && a.xs_h % 2 == 0 && a.xs_w % 2 == 0;
        hipError_t e;
        switch (d.dtype) {
        case CONV_F32: e = dwt_go<float, false>(a, grid, s); break;
        case CONV_F16: e = twx ? dwt_go<f16_t, true>(a, grid, s) : dwt_go<f16_t, false>(a, grid, s); break;
        default: e = twx ? dwt_go<bf16_t, true>(a, grid, s) : dwt_go<bf16_t, false>(a, grid, s); break;
        }
        return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
    }
    // Word loads of x: multiplier 1 with 16-bit channel pairs on 4-byte
    // boundaries of x.
    const bool wx = a.M == 1 && esize(d.dtype) == 2 && (reinterpret_cast<uintptr_t>(x) & 3) == 0 && d.C_in % 2 == 0 &&
                    a.xs_n % 2 == 0 && a.xs_h % 2 == 0 && a.xs_w % 2 == 0;
    // The multiplier schedule: 16-bit, m = 2 or 4, input channel pairs on
    // 4-byte boundaries of x and output runs of 2m channels on 4m-byte
    // boundaries of y.
    const int64_t ysa = 2 * a.M;
    const bool mult = a.ys_c == 1 && esize(d.dtype) == 2 && (a.M == 2 || a.M == 4) && d.C_in % 2 == 0 &&
                      (reinterpret_cast<uintptr_t>(x) & 3) == 0 && a.xs_n % 2 == 0 && a.xs_h % 2 == 0 &&
                      a.xs_w % 2 == 0 && (reinterpret_cast<uintptr_t>(y) & (4 * a.M - 1)) == 0 && a.ys_n % ysa == 0 &&
                      a.ys_h % ysa == 0 && a.ys_w % ysa == 0;
    if (mult) {
        DwgArgs m = a;
        m.ch_blocks = (int32_t)cdiv(d.C_in / 2, 32);
        const dim3 mgrid((unsigned)(d.N * (int64_t)a.OH * a.col_blocks * m.ch_blocks));
        const int kb = a.KW <= 3 ? 3 : (a.KW <= 5 ? 5 : 9);
        hipError_t e = hipErrorInvalidValue;
#define MICONV_DWM(MO_, KB_, S_)                                                                     \
    if (a.M == MO_ && kb == KB_ && a.SW == S_) {                                                      \
        if (d.dtype == CONV_F16)                                                                      \
            hipLaunchKernelGGL((dwm_kernel<f16_t, MO_, KB_, S_>), mgrid, dim3(256), 0, s, m);         \
        else                                                                                          \
            hipLaunchKernelGGL((dwm_kernel<bf16_t, MO_, KB_, S_>), mgrid, dim3(256), 0, s, m);        \
        e = hipGetLastError();                                                                        \
    }
        MICONV_DWM(2, 3, 1) MICONV_DWM(2, 5, 1) MICONV_DWM(2, 9, 1) MICONV_DWM(2, 3, 2) MICONV_DWM(2, 5, 2)
        MICONV_DWM(2, 9, 2) MICONV_DWM(2, 3, 3) MICONV_DWM(2, 5, 3) MICONV_DWM(2, 9, 3)
        MICONV_DWM(4, 3, 1) MICONV_DWM(4, 5, 1) MICONV_DWM(4, 9, 1) MICONV_DWM(4, 3, 2) MICONV_DWM(4, 5, 2)
        MICONV_DWM(4, 9, 2) MICONV_DWM(4, 3, 3) MICONV_DWM(4, 5, 3) MICONV_DWM(4, 9, 3)
#undef MICONV_DWM
        return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
    }
    hipError_t e;
    switch (d.dtype) {
    case CONV_F32: e = dwg_go<float, false>(a, grid, s); break;
    case CONV_F16: e = wx ? dwg_go<f16_t, true>(a, grid, s) : dwg_go<f16_t, false>(a, grid, s); break;
    default: e = wx ? dwg_go<bf16_t, true>(a, grid, s) : dwg_go<bf16_t, false>(a, grid, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

// Kernel sizes and strides with a compiled schedule (square kernels, equal strides).
bool dwcl_has_schedule(int64_t kh, int64_t kw, int64_t sh, int64_t sw)
{
    return kh == kw && sh == sw && (kh == 3 || kh == 5 || kh == 7 || kh == 9) && (sh == 1 || sh == 2);
}

int launch_dwcl(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream, bool vec)
{
    if (p.variant == DWCL_GENERIC) return launch_dwg(p, x, w, b, y, stream);
    const conv_desc &d = p.d;
    DwArgs a;
    a.x = x;
    a.w = w;
    a.b = b;
    a.y = y;
    a.xs_n = (int32_t)d.x.strides[0];
    a.xs_h = (int32_t)d.x.strides[2];
    a.xs_w = (int32_t)d.x.strides[3];
    a.x_bytes = (int32_t)p.tile[DW_XBYTES];
    a.y_bytes = (int32_t)p.tile[DW_YBYTES];
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
    a.ch_chunks = (int32_t)p.tile[DW_CHCHUNKS];
    a.col_chunks = (int32_t)p.tile[DW_COLCHUNKS];
    a.rblocks = (int32_t)p.tile[DW_RBLOCKS];
    a.rpb = (int32_t)p.tile[DW_RPB];
    a.has_bias = d.has_bias;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const int k = (int)d.k[0], st = (int)d.stride[0];
    const int64_t grid = p.grid[0];
    // 16-byte loads and stores need 16-byte aligned channel runs (the plan's
    // variant 1) and 16-byte aligned x and y.
    const bool q = p.variant == 1 && vec;
    switch (d.dtype) {
    case CONV_F32: e = q ? dispatch<float, 16>(a, grid, k, st, s) : dispatch<float, 4>(a, grid, k, st, s); break;
    case CONV_F16: e = q ? dispatch<f16_t, 16>(a, grid, k, st, s) : dispatch<f16_t, 4>(a, grid, k, st, s); break;
    default: e = q ? dispatch<bf16_t, 16>(a, grid, k, st, s) : dispatch<bf16_t, 4>(a, grid, k, st, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
