// Weight and bias gradients of the canonical op (conv_run_backward).
//
// torch/_inductor/kernel/conv.py (convolution_backward): the weight gradient
// is a GEMM whose reduction runs over images and positions, and the bias
// gradient sums the output gradient over them.  For the forward op the
// terms are x[n, ci, o*s - pb + t*dil] * w[co, c, t]; for the transposed op
// x[n, ci, i] * w[ci, j, t] with output position o = i*s - pb + t*dil.  In
// both the weight gradient reads one dense operand P over a set of
// positions m and one operand Q gathered at m*s - pb + t*dil:
//
//   dW[g*PC + a, b, t] = sum_m P[n, g*PC + a, m] * Q[n, g*QC + b, m*s - pb + t*dil]
//
//   forward:    P = gy (positions: y's), Q = x  (zero outside x),  PC = Cog, QC = Cig
//   transposed: P = x  (positions: x's), Q = gy (zero outside y),  PC = Cig, QC = Cog
//
// which is exactly the weight layout of each op ([C_out, Cig, k] forward,
// [C_in, Cog, k] transposed: first index g*PC + a, second b).
//
// Kernels
//   wgrad_mfma    16-bit, channel-contiguous P and Q in 16-byte chunks: a
//                 workgroup owns (group, tap, 128 a x 128 b) and one range of
//                 m; per 32-position step it loads [32 m x 128 ch] of each
//                 operand (16-byte chunks of 8 channels) and writes them
//                 transposed into LDS as [ch][m], so the MFMA operands hold 8
//                 consecutive positions per lane (v_mfma_f32_16x16x32); the
//                 next step's chunks are loaded into registers while the
//                 current one is multiplied.
//   wgrad_simple  any dtype and layout: one thread per weight element and
//                 range of m, fp32 sums.
//   wgrad_plane   few channels per group, channel-major x and gy: a workgroup
//                 per (group, range of images) stages each image's planes in
//                 LDS; a thread per (out channel, in channel, tap) walks them.
//   wgrad_dw      depthwise, 16-bit, channels-last x and gy: a workgroup owns
//                 256/TG channel words and one range of rows (n, output
//                 row); thread = one channel word x one of TG tap groups (taps
//                 tg, tg + TG, ...; TG = 2, 4 or 8 by kernel size), looping over
//                 the row's positions: one gy word, then one x word per tap,
//                 two fp32 FMAs each.
//   bgrad         per-channel sums of gy over one range of positions.
//   gy_to_cl      a channel-major 16-bit gy copied channels-last through LDS
//                 tiles, so the gradients of a channels-last call read both
//                 operands in 16-byte channel chunks.
//   bwd_reduce    sums the fp32 partial sums of the ranges (64 outputs x 4
//                 interleaved quarters of the ranges per workgroup), rounds
//                 once to the dtype and stores at the gradient's strides.
#include "dev_common.h"
#include "internal.h"

#include <algorithm>
#include <cstring>

namespace miconv {

struct WgArgs {
    const void *P;
    const void *Q;
    float *part;                 // [S][G][T][apad][bpad] partial sums
    int64_t ps_n, ps_c, ps_l[3]; // element strides of P
    int64_t qs_n, qs_c, qs_l[3]; // element strides of Q
    int32_t N, G, PC, QC, T, apad, bpad;
    int32_t E[3];                // P's spatial extents (positions m)
    int32_t F[3];                // Q's spatial extents
    int32_t K[3], S[3], PB[3], D[3];
    int32_t PH2, PW2;            // padding after in slots 1 and 2 (the plane schedule's halo)
    int32_t splits;              // ranges of m
    int64_t M;                   // N * E0 * E1 * E2
    int32_t p_bytes, q_bytes;    // buffer ranges (16-byte path)
};

namespace {

// Position m -> (n, e0, e1, e2).
__device__ __forceinline__ void split_m(int64_t m, const WgArgs &a, int &n, int &e0, int &e1, int &e2)
{
    const int64_t E12 = (int64_t)a.E[1] * a.E[2];
    const int64_t per = E12 * a.E[0];
    n = (int)(m / per);
    const int64_t r = m - (int64_t)n * per;
    e0 = (int)(r / E12);
    const int64_t r2 = r - (int64_t)e0 * E12;
    e1 = (int)(r2 / a.E[2]);
    e2 = (int)(r2 - (int64_t)e1 * a.E[2]);
}

// Range [m_lo, m_hi) of split `sp`, in whole 32-position steps.
__device__ __forceinline__ void m_range(const WgArgs &a, int sp, int64_t &lo, int64_t &hi)
{
    const int64_t steps = (a.M + 31) / 32;
    lo = steps * sp / a.splits * 32;
    hi = std::min<int64_t>(steps * (sp + 1) / a.splits * 32, a.M);
}

// LDS offset of 16-byte chunk c (8 positions) of channel row r, rows of 32
// positions: rows are 64 bytes, every 8 rows one spare row so that rows r
// and r + 8 use opposite halves of the banks, and the chunk is XORed with
// bits 1-2 of the row, so the 8 lanes of one ds_read_b128 cycle (8
// consecutive rows, one chunk) hit 8 different 16-byte bank groups.
__device__ __forceinline__ int wg_off(int r, int c) { return (r + (r >> 3)) * 64 + ((c ^ ((r >> 1) & 3)) * 16); }

}  // namespace

constexpr int WG_TILE = 128;
constexpr int WG_ROWS = WG_TILE + WG_TILE / 8;   // LDS rows per operand with the spare rows

// PM_P / PM_Q: that operand is read position-major (8 consecutive positions
// of one channel per chunk, gathered element by element: any strides, the
// last spatial extent a multiple of 8 so a chunk stays in one row) instead of
// channel-major (16-byte chunks of 8 channels at one position, transposed on
// the way into LDS).
template <typename T, bool PM_P, bool PM_Q>
__global__ __launch_bounds__(256) void wgrad_mfma_kernel(WgArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ __attribute__((aligned(16))) unsigned char sm[2][2][WG_ROWS * 64];   // [buffer][P/Q]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Block order (fastest first): split, b tile, a tile, tap, group.
    int blk = blockIdx.x;
    const int sp = blk % a.splits;
    blk /= a.splits;
    const int btiles = a.bpad / WG_TILE, atiles = a.apad / WG_TILE;
    const int bt = blk % btiles;
    blk /= btiles;
    const int at = blk % atiles;
    blk /= atiles;
    const int t = blk % a.T;
    const int g = blk / a.T;
    const int t2 = t % a.K[2], t1 = (t / a.K[2]) % a.K[1], t0 = t / (a.K[2] * a.K[1]);
    const int toff0 = t0 * a.D[0] - a.PB[0], toff1 = t1 * a.D[1] - a.PB[1], toff2 = t2 * a.D[2] - a.PB[2];

    int64_t m_lo, m_hi;
    m_range(a, sp, m_lo, m_hi);

    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.P), (short)0, a.p_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t qr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.Q), (short)0, a.q_bytes, 0x00020000);
    const T *__restrict__ Pe = static_cast<const T *>(a.P);
    const T *__restrict__ Qe = static_cast<const T *>(a.Q);
    const int a0 = at * WG_TILE, b0 = bt * WG_TILE;
    // Registers of the next step: per operand two 16-byte chunks.  Channel
    // mode: thread -> position lm = tid & 31 and channel chunks (tid >> 5) and
    // (tid >> 5) + 8.  Position mode: chunk id tid + 256h -> 8-position block
    // (id & 3) of channel (id >> 2).
    const int lm = tid & 31, lc = tid >> 5;
    uint4 rp[2], rq[2];
    auto gload = [&](int64_t mbase) {
        // Channel-major chunks of both operands at position mbase + lm.
        if constexpr (!PM_P || !PM_Q) {
            const int64_t m = mbase + lm;
            int n = 0, e0 = 0, e1 = 0, e2 = 0;
            const bool live = m < m_hi;
            if (live) split_m(m, a, n, e0, e1, e2);
            const int64_t pbase = (int64_t)n * a.ps_n + e0 * a.ps_l[0] + e1 * a.ps_l[1] + e2 * a.ps_l[2];
            const int q0 = e0 * a.S[0] + toff0, q1 = e1 * a.S[1] + toff1, q2 = e2 * a.S[2] + toff2;
            const bool qin = live && (unsigned)q0 < (unsigned)a.F[0] && (unsigned)q1 < (unsigned)a.F[1] &&
                             (unsigned)q2 < (unsigned)a.F[2];
            const int64_t qbase = (int64_t)n * a.qs_n + q0 * a.qs_l[0] + q1 * a.qs_l[1] + q2 * a.qs_l[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ch = 8 * (lc + 8 * h);
                if constexpr (!PM_P) {
                    const bool pok = live && a0 + ch < a.PC;
                    const int po = pok ? (int)((pbase + (int64_t)(g * a.PC + a0 + ch) * a.ps_c) * 2) : 0x7fffff00;
                    rp[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pr, po, 0, 0));
                }
                if constexpr (!PM_Q) {
                    const bool qok = qin && b0 + ch < a.QC;
                    const int qo = qok ? (int)((qbase + (int64_t)(g * a.QC + b0 + ch) * a.qs_c) * 2) : 0x7fffff00;
                    rq[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, qo, 0, 0));
                }
            }
        }
        // Position-major chunks: 8 consecutive positions of one channel, all
        // in one row of the last spatial dim.
        if constexpr (PM_P || PM_Q) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int id = tid + 256 * h, blk8 = id & 3, ch = id >> 2;
                const int64_t m = mbase + 8 * blk8;
                int n = 0, e0 = 0, e1 = 0, e2 = 0;
                const bool live = m < m_hi;
                if (live) split_m(m, a, n, e0, e1, e2);
                uint16_t v[8];
                if constexpr (PM_P) {
                    const bool ok = live && a0 + ch < a.PC;
                    const int64_t base = (int64_t)n * a.ps_n + (int64_t)(g * a.PC + a0 + ch) * a.ps_c +
                                         e0 * a.ps_l[0] + e1 * a.ps_l[1] + e2 * a.ps_l[2];
                    const int64_t st = a.ps_l[2];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const T val = (ok && m + e < m_hi) ? Pe[base + e * st] : T{};
                        __builtin_memcpy(&v[e], &val, 2);
                    }
                    __builtin_memcpy(&rp[h], v, 16);
                }
                if constexpr (PM_Q) {
                    const bool ok = live && b0 + ch < a.QC;
                    const int q0 = e0 * a.S[0] + toff0, q1 = e1 * a.S[1] + toff1;
                    const bool rowin = ok && (unsigned)q0 < (unsigned)a.F[0] && (unsigned)q1 < (unsigned)a.F[1];
                    const int64_t base = (int64_t)n * a.qs_n + (int64_t)(g * a.QC + b0 + ch) * a.qs_c +
                                         q0 * a.qs_l[0] + q1 * a.qs_l[1];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int q2 = (e2 + e) * a.S[2] + toff2;
                        const bool in = rowin && m + e < m_hi && (unsigned)q2 < (unsigned)a.F[2];
                        const T val = in ? Qe[base + (int64_t)q2 * a.qs_l[2]] : T{};
                        __builtin_memcpy(&v[e], &val, 2);
                    }
                    __builtin_memcpy(&rq[h], v, 16);
                }
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (!PM_P || !PM_Q) {
                // Channel-major chunk: element e is channel ch + e at position lm.
                const int ch = 8 * (lc + 8 * h);
                uint16_t vp[8], vq[8];
                __builtin_memcpy(vp, &rp[h], 16);
                __builtin_memcpy(vq, &rq[h], 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int off = wg_off(ch + e, lm >> 3) + (lm & 7) * 2;
                    if constexpr (!PM_P) *reinterpret_cast<uint16_t *>(&sm[buf][0][off]) = vp[e];
                    if constexpr (!PM_Q) *reinterpret_cast<uint16_t *>(&sm[buf][1][off]) = vq[e];
                }
            }
            if constexpr (PM_P || PM_Q) {
                const int id = tid + 256 * h, blk8 = id & 3, ch = id >> 2;
                if constexpr (PM_P) *reinterpret_cast<uint4 *>(&sm[buf][0][wg_off(ch, blk8)]) = rp[h];
                if constexpr (PM_Q) *reinterpret_cast<uint4 *>(&sm[buf][1][wg_off(ch, blk8)]) = rq[h];
            }
        }
    };

    const int wa = wave >> 1, wb = wave & 1;   // wave tile: a rows 64*wa.., b rows 64*wb..
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
        uint4 af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const uint4 *>(&sm[buf][0][wg_off(64 * wa + 16 * i + lr, lg)]);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const uint4 *>(&sm[buf][1][wg_off(64 * wb + 16 * j + lr, lg)]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma_16x16x32(af[i], bf[j], acc[i][j], T{});
    };

    const int nsteps = (int)((m_hi - m_lo + 31) / 32);
    if (nsteps > 0) {
        gload(m_lo);
        sstore(0);
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            const bool more = s + 1 < nsteps;
            if (more) gload(m_lo + 32 * (s + 1));
            compute(s & 1);
            if (more) sstore((s + 1) & 1);
            __syncthreads();
        }
    }
    // Partial sums of this range: lane holds a rows 64*wa + 16i + 4*lg + e of
    // b column 64*wb + 16j + lr.
    float *Pt = a.part + ((((int64_t)sp * a.G + g) * a.T + t) * a.apad) * a.bpad;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ar = a0 + 64 * wa + 16 * i + 4 * lg + e, bc = b0 + 64 * wb + 16 * j + lr;
                Pt[(int64_t)ar * a.bpad + bc] = acc[i][j][e];
            }
#endif
}

// One thread per (group, tap, a, b) and range of m, fp32 sum.
template <typename T>
__global__ __launch_bounds__(256) void wgrad_simple_kernel(WgArgs a)
{
    const int64_t per = (int64_t)a.G * a.T * a.PC * a.QC;
    const int64_t total = per * a.splits;
    const T *__restrict__ P = static_cast<const T *>(a.P);
    const T *__restrict__ Q = static_cast<const T *>(a.Q);
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int sp = (int)(idx / per);
        int64_t r = idx - sp * per;
        const int b = (int)(r % a.QC);
        r /= a.QC;
        const int av = (int)(r % a.PC);
        r /= a.PC;
        const int t = (int)(r % a.T);
        const int g = (int)(r / a.T);
        const int t2 = t % a.K[2], t1 = (t / a.K[2]) % a.K[1], t0 = t / (a.K[2] * a.K[1]);
        int64_t lo, hi;
        m_range(a, sp, lo, hi);
        float sum = 0.f;
        for (int64_t m = lo; m < hi; ++m) {
            int n, e0, e1, e2;
            split_m(m, a, n, e0, e1, e2);
            const int q0 = e0 * a.S[0] - a.PB[0] + t0 * a.D[0];
            const int q1 = e1 * a.S[1] - a.PB[1] + t1 * a.D[1];
            const int q2 = e2 * a.S[2] - a.PB[2] + t2 * a.D[2];
            if ((unsigned)q0 >= (unsigned)a.F[0] || (unsigned)q1 >= (unsigned)a.F[1] || (unsigned)q2 >= (unsigned)a.F[2])
                continue;
            const float pv = to_f32(P[(int64_t)n * a.ps_n + (int64_t)(g * a.PC + av) * a.ps_c + e0 * a.ps_l[0] +
                                      e1 * a.ps_l[1] + e2 * a.ps_l[2]]);
            const float qv = to_f32(Q[(int64_t)n * a.qs_n + (int64_t)(g * a.QC + b) * a.qs_c + q0 * a.qs_l[0] +
                                      q1 * a.qs_l[1] + q2 * a.qs_l[2]]);
            sum = fmaf(pv, qv, sum);
        }
        a.part[((((int64_t)sp * a.G + g) * a.T + t) * a.apad + av) * a.bpad + b] = sum;
    }
}

struct BgArgs {
    const void *gy;
    float *part;                 // [S][C] partial sums
    int64_t gs_n, gs_c, gs_l[3];
    int32_t N, C, O[3], splits;
    int64_t M;                   // N * O0 * O1 * O2
};

// Block (split, 64-channel chunk): 4 groups of 64 threads, thread = channel;
// the groups take consecutive quarters of the split's range of positions.
// Channel-fastest lanes read consecutive channels of one position
// (channels-last gy); the partial sums of the 4 groups are added in LDS.
template <typename T>
__global__ __launch_bounds__(256) void bgrad_kernel(BgArgs a)
{
    __shared__ float red[4][64];
    const int chunks = (a.C + 63) / 64;
    const int sp = blockIdx.x / chunks, ck = blockIdx.x % chunks;
    const int c = ck * 64 + (threadIdx.x & 63), grp = threadIdx.x >> 6;
    const int64_t per = (a.M + a.splits - 1) / a.splits;
    const int64_t lo0 = per * sp, hi0 = std::min<int64_t>(lo0 + per, a.M);
    // The four wave groups take consecutive quarters of the range, so each
    // lane walks its positions in order: the position is decomposed once and
    // then advanced (no division per element); the 64 lanes of a wave read
    // 64 channels of one position, 16 positions in flight.
    const int64_t q = (std::max<int64_t>(hi0 - lo0, 0) + 3) / 4;
    const int64_t lo = std::min<int64_t>(lo0 + q * grp, hi0), hi = std::min<int64_t>(lo + q, hi0);
    const T *__restrict__ G = static_cast<const T *>(a.gy);
    const int64_t O12 = (int64_t)a.O[1] * a.O[2], O012 = O12 * a.O[0];
    float sum = 0.f;
    if (c < a.C && lo < hi) {
        const int64_t n = lo / O012, r = lo - n * O012;
        int o0 = (int)(r / O12);
        const int64_t r2 = r - (int64_t)o0 * O12;
        int o1 = (int)(r2 / a.O[2]), o2 = (int)(r2 - (int64_t)o1 * a.O[2]);
        int64_t off = n * a.gs_n + (int64_t)c * a.gs_c + o0 * a.gs_l[0] + o1 * a.gs_l[1] + o2 * a.gs_l[2];
        auto advance = [&]() {
            if (++o2 < a.O[2]) { off += a.gs_l[2]; return; }
            o2 = 0;
            off -= (int64_t)(a.O[2] - 1) * a.gs_l[2];
            if (++o1 < a.O[1]) { off += a.gs_l[1]; return; }
            o1 = 0;
            off -= (int64_t)(a.O[1] - 1) * a.gs_l[1];
            if (++o0 < a.O[0]) { off += a.gs_l[0]; return; }
            o0 = 0;
            off += a.gs_n - (int64_t)(a.O[0] - 1) * a.gs_l[0];
        };
        int64_t m = lo;
        constexpr int LU = 16;   // loads in flight before the adds
        for (; m + LU <= hi; m += LU) {
            T v[LU];
#pragma unroll
            for (int u = 0; u < LU; ++u) {
                v[u] = G[off];
                advance();
            }
#pragma unroll
            for (int u = 0; u < LU; ++u) sum += to_f32(v[u]);
        }
        for (; m < hi; ++m) {
            sum += to_f32(G[off]);
            advance();
        }
    }
    red[grp][threadIdx.x & 63] = sum;
    __syncthreads();
    if (grp == 0 && c < a.C)
        a.part[(int64_t)sp * a.C + c] = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] +
                                        red[3][threadIdx.x];
}

struct RdArgs {
    const float *part;
    void *out;
    int64_t count;               // elements of the gradient
    int64_t plane;               // floats per split
    int32_t splits;
    // gradient element e -> (g, t, a, b) for the weight gradient; -> c for db
    int32_t is_w, G, T, PC, QC, apad, bpad, K1, K2;
    int64_t os0, os1, osk[3];    // the gradient's strides (weight: [g*PC + a, b, k...]; db: os0)
};

template <typename T>
// Lane (o, q) of a workgroup: output e = 64 * block + o, summing the ranges
// k = q, q + 4, ... with four independent partial sums (loads in flight);
// the four quarter sums meet in LDS and lane q = 0 rounds once and stores.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(RdArgs a)
{
    __shared__ float red[4][64];
    T *__restrict__ out = static_cast<T *>(a.out);
    const int o = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.x * 64 + o;
    int64_t src = 0, dst = 0;
    if (e < a.count) {
        if (a.is_w) {
            int64_t r = e;
            const int b = (int)(r % a.QC);
            r /= a.QC;
            const int av = (int)(r % a.PC);
            r /= a.PC;
            const int t = (int)(r % a.T);
            const int g = (int)(r / a.T);
            src = (((int64_t)g * a.T + t) * a.apad + av) * a.bpad + b;
            const int t2 = t % a.K2, t1 = (t / a.K2) % a.K1, t0 = t / (a.K2 * a.K1);
            dst = (int64_t)(g * a.PC + av) * a.os0 + (int64_t)b * a.os1 + t0 * a.osk[0] + t1 * a.osk[1] +
                  t2 * a.osk[2];
        } else {
            src = e;
            dst = e * a.os0;
        }
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        const float *p = a.part + src;
        int k = q;
        for (; k + 12 < a.splits; k += 16) {
            s0 += p[(int64_t)k * a.plane];
            s1 += p[(int64_t)(k + 4) * a.plane];
            s2 += p[(int64_t)(k + 8) * a.plane];
            s3 += p[(int64_t)(k + 12) * a.plane];
        }
        for (; k < a.splits; k += 4) s0 += p[(int64_t)k * a.plane];
        red[q][o] = (s0 + s1) + (s2 + s3);
    }
    __syncthreads();
    if (q == 0 && e < a.count) out[dst] = from_f32<T>((red[0][o] + red[1][o]) + (red[2][o] + red[3][o]));
}

namespace {

// Depthwise weight gradient, channel words: dw[c, t] = sum over (n, e1, e2)
// of gy[n, e1, e2, c] * x[n, e1*S1 - PB1 + kh*D1, e2*S2 - PB2 + kw*D2, c] for
// tap t = (kh, kw), in the slots 1 and 2 of WgArgs (slot 0 has extent 1).
// Partial sums per range of rows go to part[sp][c][t] (apad = bpad = 1).
template <typename T, int MT, int TG>
__global__ __launch_bounds__(256) void wgrad_dw_kernel(WgArgs a)
{
    constexpr int WPG = 256 / TG;                // channel words of the workgroup
    const int tid = threadIdx.x;
    const int wd = tid % WPG, tg = tid / WPG;
    const int cchunks = (a.G + 2 * WPG - 1) / (2 * WPG);
    const int cc = blockIdx.x % cchunks, sp = blockIdx.x / cchunks;
    const int word = cc * WPG + wd;
    const bool cok = 2 * word < a.G;
    const int KW = a.K[2];
    int dh[MT], dwo[MT];
    bool tv[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int t = tg + TG * j;
        tv[j] = t < a.T;
        dh[j] = tv[j] ? (t / KW) * a.D[1] : 0;
        dwo[j] = tv[j] ? (t % KW) * a.D[2] : 0;
    }
    float acc[MT][2];
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[j][0] = acc[j][1] = 0.f;
    const int64_t rows = (int64_t)a.N * a.E[1];
    const int64_t r0 = rows * sp / a.splits, r1 = rows * (sp + 1) / a.splits;
    const uint32_t *P = static_cast<const uint32_t *>(a.P);
    const uint32_t *Q = static_cast<const uint32_t *>(a.Q);
    for (int64_t r = r0; r < r1 && cok; ++r) {
        const int n = (int)(r / a.E[1]), e1 = (int)(r % a.E[1]);
        const int64_t pbase = ((int64_t)n * a.ps_n + (int64_t)e1 * a.ps_l[1]) / 2 + word;
        const int ih0 = e1 * a.S[1] - a.PB[1];
        int64_t qrow[MT];
        bool hok[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int ih = ih0 + dh[j];
            hok[j] = tv[j] && (unsigned)ih < (unsigned)a.F[1];
            qrow[j] = hok[j] ? ((int64_t)n * a.qs_n + (int64_t)ih * a.qs_l[1]) / 2 + word : 0;
        }
        // PU positions per pass: all their loads in flight before the FMAs.
        constexpr int PU = MT <= 4 ? 4 : 2;
        for (int e2b = 0; e2b < a.E[2]; e2b += PU) {
            uint32_t g[PU], xv[PU][MT];
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const int e2 = e2b + u;
                const bool pok = e2 < a.E[2];
                g[u] = pok ? P[pbase + (int64_t)e2 * (a.ps_l[2] / 2)] : 0u;
                const int iw0 = e2 * a.S[2] - a.PB[2];
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    const int iw = iw0 + dwo[j];
                    const bool ok = pok && hok[j] && (unsigned)iw < (unsigned)a.F[2];
                    xv[u][j] = ok ? Q[qrow[j] + (int64_t)iw * (a.qs_l[2] / 2)] : 0u;
                }
            }
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const float g0 = lo_f32(g[u], T{}), g1 = hi_f32(g[u], T{});
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    acc[j][0] = __builtin_fmaf(g0, lo_f32(xv[u][j], T{}), acc[j][0]);
                    acc[j][1] = __builtin_fmaf(g1, hi_f32(xv[u][j], T{}), acc[j][1]);
                }
            }
        }
    }
    if (!cok) return;
    float *part = a.part + (int64_t)sp * a.G * a.T;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        if (!tv[j]) continue;
        const int t = tg + TG * j;
        part[(int64_t)(2 * word) * a.T + t] = acc[j][0];
        part[(int64_t)(2 * word + 1) * a.T + t] = acc[j][1];
    }
}

// Few-channel grouped weight gradient on channel-major operands (forward
// calls, rank <= 2 in slots 1 and 2 of WgArgs): workgroup = (group g, range of
// images).  Per image, the group's QC x planes land in LDS as fp32 inside a
// zero halo of the padding, and its PC gy planes beside them; thread j walks
// the (a, b, t) = (output channel, input channel, tap) elements j, j + 256,
// ... and, per element, every position:
//   dw[g*PC + a, b, t] += gy[a, e1, e2] * xh[b, e1*S1 + kh*D1, e2*S2 + kw*D2].
// fp32 partial sums per range of images go to part[sp][g][t][a][b].
template <typename T>
__global__ __launch_bounds__(256) void wgrad_plane_kernel(WgArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float wl[];
    const int g = blockIdx.x % a.G, sp = blockIdx.x / a.G;
    const int E1 = a.E[1], E2 = a.E[2];
    const int HH = a.F[1] + a.PB[1] + a.PH2, WW = a.F[2] + a.PB[2] + a.PW2;   // haloed x plane
    float *gyl = wl;                                  // [PC][E1][E2]
    float *xl = wl + a.PC * E1 * E2;                  // [QC][HH][WW]
    const int EL = a.PC * a.QC * a.T;                 // elements of the group's gradient
    const int n0 = (int)((int64_t)a.N * sp / a.splits), n1 = (int)((int64_t)a.N * (sp + 1) / a.splits);
    const T *__restrict__ P = static_cast<const T *>(a.P);
    const T *__restrict__ Q = static_cast<const T *>(a.Q);
    const int KW = a.K[2];
    float acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = 0.f;
    for (int n = n0; n < n1; ++n) {
        __syncthreads();   // the previous image's planes are no longer read
        for (int i = threadIdx.x; i < a.PC * E1 * E2; i += 256) {
            const int c = i / (E1 * E2), pos = i - c * (E1 * E2);
            const int e1 = pos / E2, e2 = pos - e1 * E2;
            gyl[i] = to_f32(P[(int64_t)n * a.ps_n + (int64_t)(g * a.PC + c) * a.ps_c + (int64_t)e1 * a.ps_l[1] +
                              (int64_t)e2 * a.ps_l[2]]);
        }
        for (int i = threadIdx.x; i < a.QC * HH * WW; i += 256) {
            const int c = i / (HH * WW), pos = i - c * (HH * WW);
            const int h = pos / WW - a.PB[1], w = pos % WW - a.PB[2];
            float v = 0.f;
            if ((unsigned)h < (unsigned)a.F[1] && (unsigned)w < (unsigned)a.F[2])
                v = to_f32(Q[(int64_t)n * a.qs_n + (int64_t)(g * a.QC + c) * a.qs_c + (int64_t)h * a.qs_l[1] +
                             (int64_t)w * a.qs_l[2]]);
            xl[i] = v;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int el = threadIdx.x + r * 256;
            if (el >= EL) break;
            const int t = el % a.T, ab = el / a.T;
            const int bi = ab % a.QC, ai = ab / a.QC;
            const int kh = t / KW, kw = t % KW;
            const float *gp = gyl + ai * E1 * E2;
            const float *xp = xl + bi * HH * WW + kh * a.D[1] * WW + kw * a.D[2];
            float s = 0.f;
            for (int e1 = 0; e1 < E1; ++e1) {
                const float *gr = gp + e1 * E2;
                const float *xr = xp + e1 * a.S[1] * WW;
                for (int e2 = 0; e2 < E2; ++e2) s = __builtin_fmaf(gr[e2], xr[e2 * a.S[2]], s);
            }
            acc[r] += s;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int el = threadIdx.x + r * 256;
        if (el >= EL) break;
        const int t = el % a.T, ab = el / a.T;
        const int bi = ab % a.QC, ai = ab / a.QC;
        a.part[(((int64_t)sp * a.G + g) * a.T + t) * a.apad * a.bpad + (int64_t)ai * a.bpad + bi] = acc[r];
    }
}

template <typename T>
hipError_t launch_wgrad_dw(const WgArgs &a, hipStream_t s)
{
    if constexpr (Dt<T>::size == 2) {
        const int tg = wgrad_dw_tg(a.T);
        const dim3 blocks((unsigned)(((a.G + 2 * (256 / tg) - 1) / (2 * (256 / tg))) * (int64_t)a.splits));
        const int mt = (a.T + tg - 1) / tg;
        if (tg == 2 && mt <= 5) hipLaunchKernelGGL((wgrad_dw_kernel<T, 5, 2>), blocks, dim3(256), 0, s, a);
        else if (tg == 2 && mt <= 8) hipLaunchKernelGGL((wgrad_dw_kernel<T, 8, 2>), blocks, dim3(256), 0, s, a);
        else if (tg == 4 && mt <= 7) hipLaunchKernelGGL((wgrad_dw_kernel<T, 7, 4>), blocks, dim3(256), 0, s, a);
        else if (tg == 8 && mt <= 7) hipLaunchKernelGGL((wgrad_dw_kernel<T, 7, 8>), blocks, dim3(256), 0, s, a);
        else if (tg == 8 && mt <= 11) hipLaunchKernelGGL((wgrad_dw_kernel<T, 11, 8>), blocks, dim3(256), 0, s, a);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_wgrad_t(const WgArgs &a, bool mfma, bool pm_p, bool pm_q, hipStream_t s)
{
    if constexpr (Dt<T>::size == 2) {
        if (mfma) {
            const dim3 blocks(a.G * a.T * (a.apad / WG_TILE) * (a.bpad / WG_TILE) * a.splits);
            if (!pm_p && !pm_q) hipLaunchKernelGGL((wgrad_mfma_kernel<T, false, false>), blocks, dim3(256), 0, s, a);
            else if (pm_p && !pm_q) hipLaunchKernelGGL((wgrad_mfma_kernel<T, true, false>), blocks, dim3(256), 0, s, a);
            else if (!pm_p && pm_q) hipLaunchKernelGGL((wgrad_mfma_kernel<T, false, true>), blocks, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((wgrad_mfma_kernel<T, true, true>), blocks, dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    {
        const int64_t total = (int64_t)a.G * a.T * a.PC * a.QC * a.splits;
        const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 65536);
        hipLaunchKernelGGL((wgrad_simple_kernel<T>), dim3(blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_t(const RdArgs &r, hipStream_t s)
{
    const unsigned blocks = (unsigned)cdiv(r.count, 64);
    hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3(blocks), dim3(256), 0, s, r);
    return hipGetLastError();
}

// Position-contiguous gy (channel-major, every image's channel plane one
// run): block (n, c) sums the run of positions of one plane, lanes on
// consecutive positions, into part[n][c] (the ranges are the images).
template <typename T>
__global__ __launch_bounds__(256) void bgrad_rows_kernel(BgArgs a)
{
    __shared__ float red[256];
    const int c = blockIdx.x % a.C, n = blockIdx.x / a.C;
    const int64_t L = (int64_t)a.O[0] * a.O[1] * a.O[2];
    const T *__restrict__ G = static_cast<const T *>(a.gy) + (int64_t)n * a.gs_n + (int64_t)c * a.gs_c;
    float s0 = 0.f, s1 = 0.f;
    int64_t i = threadIdx.x;
    for (; i + 256 < L; i += 512) {
        s0 += to_f32(G[i]);
        s1 += to_f32(G[i + 256]);
    }
    if (i < L) s0 += to_f32(G[i]);
    red[threadIdx.x] = s0 + s1;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.part[(int64_t)n * a.C + c] = red[0];
}

template <typename T>
hipError_t launch_bgrad_t(const BgArgs &b, bool rows, hipStream_t s)
{
    if (rows) {
        hipLaunchKernelGGL((bgrad_rows_kernel<T>), dim3((unsigned)((int64_t)b.N * b.C)), dim3(256), 0, s, b);
        return hipGetLastError();
    }
    const int blocks = b.splits * (int)cdiv(b.C, 64);
    hipLaunchKernelGGL((bgrad_kernel<T>), dim3(blocks), dim3(256), 0, s, b);
    return hipGetLastError();
}

}  // namespace

// Zeros at a tensor's strides (a gradient with no terms).
template <typename T>
__global__ void fill_zero_kernel(T *out, int64_t count, int rank, int64_t s0, int64_t s1, int64_t s2, int64_t s3,
                                 int64_t s4, int64_t z1, int64_t z2, int64_t z3, int64_t z4)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = e, off = 0;
        const int64_t sz[5] = {0, z1, z2, z3, z4}, st[5] = {s0, s1, s2, s3, s4};
        for (int i = rank - 1; i >= 1; --i) {
            off += (r % sz[i]) * st[i];
            r /= sz[i];
        }
        off += r * st[0];
        out[off] = from_f32<T>(0.f);
    }
}

int launch_fill_zero(void *out, const conv_tensor &t, void *stream)
{
    int64_t count = 1;
    for (int i = 0; i < t.rank; ++i) count *= t.sizes[i];
    if (count == 0) return CONV_OK;
    int64_t sz[5] = {1, 1, 1, 1, 1}, st[5] = {0, 0, 0, 0, 0};
    for (int i = 0; i < t.rank; ++i) {
        sz[i] = t.sizes[i];
        st[i] = t.strides[i];
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(count, 256), 8192);
    switch (t.dtype) {
    case CONV_F32:
        hipLaunchKernelGGL((fill_zero_kernel<float>), dim3(blocks), dim3(256), 0, s, static_cast<float *>(out), count,
                           t.rank, st[0], st[1], st[2], st[3], st[4], sz[1], sz[2], sz[3], sz[4]);
        break;
    case CONV_F16:
        hipLaunchKernelGGL((fill_zero_kernel<f16_t>), dim3(blocks), dim3(256), 0, s, static_cast<f16_t *>(out), count,
                           t.rank, st[0], st[1], st[2], st[3], st[4], sz[1], sz[2], sz[3], sz[4]);
        break;
    default:
        hipLaunchKernelGGL((fill_zero_kernel<bf16_t>), dim3(blocks), dim3(256), 0, s, static_cast<bf16_t *>(out),
                           count, t.rank, st[0], st[1], st[2], st[3], st[4], sz[1], sz[2], sz[3], sz[4]);
        break;
    }
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

// The stride-1 input gradient's weight: element (ci, o, t0, t1) of the
// contiguous [C_in][Cog][K0][K1] copy is w[g*Cog + o][i][K0-1-t0][K1-1-t1]
// with ci = g*Cig + i (K1 = 1 for 1-D), bits copied unchanged.
template <typename U>
__global__ void flip_weight_kernel(const U *__restrict__ w, U *__restrict__ out, int64_t count, int32_t Cig,
                                   int32_t Cog, int32_t K0, int32_t K1, int64_t ws0, int64_t ws1, int64_t ws2,
                                   int64_t ws3)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = e;
        const int t1 = (int)(r % K1);
        r /= K1;
        const int t0 = (int)(r % K0);
        r /= K0;
        const int o = (int)(r % Cog);
        const int64_t ci = r / Cog;
        const int64_t g = ci / Cig, i = ci % Cig;
        out[e] = w[(g * Cog + o) * ws0 + i * ws1 + (int64_t)(K0 - 1 - t0) * ws2 + (int64_t)(K1 - 1 - t1) * ws3];
    }
}

int launch_flip_weight(const conv_bwd_plan_t &p, const void *w, void *dst, void *stream)
{
    const conv_desc &d = p.d;
    const bool two = d.spatial == 2;
    const int32_t Cig = (int32_t)(d.C_in / d.groups), Cog = (int32_t)(d.C_out / d.groups);
    const int32_t K0 = (int32_t)d.k[0], K1 = two ? (int32_t)d.k[1] : 1;
    const int64_t count = d.C_in * (int64_t)Cog * K0 * K1;
    if (count == 0) return CONV_OK;
    const int64_t ws2 = d.w.strides[2], ws3 = two ? d.w.strides[3] : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(count, 256), 4096);
    if (esize(d.dtype) == 4)
        hipLaunchKernelGGL((flip_weight_kernel<uint32_t>), dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint32_t *>(w), static_cast<uint32_t *>(dst), count, Cig, Cog, K0, K1,
                           d.w.strides[0], d.w.strides[1], ws2, ws3);
    else
        hipLaunchKernelGGL((flip_weight_kernel<uint16_t>), dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(w), static_cast<uint16_t *>(dst), count, Cig, Cog, K0, K1,
                           d.w.strides[0], d.w.strides[1], ws2, ws3);
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

// A channel-major 16-bit gy (image stride gs0, channel stride gs1, each
// (image, channel) plane a dense run of L positions) copied to the dense
// channels-last [N][L][C]: a workgroup moves a 128-channel x 64-position
// tile of one image through LDS, reading runs of 64 positions (128 bytes per
// wave row) and writing runs of 128 channels as channel pairs (256 bytes per
// wave row).  Channel tiles are the fastest grid dimension, so neighbouring
// workgroups complete the same output rows.  Rows of 66 elements (33 words)
// keep the column reads on distinct banks.  C is even.
__global__ __launch_bounds__(256) void gy_to_cl_kernel(const uint16_t *__restrict__ gy, uint16_t *__restrict__ out,
                                                        int64_t L, int32_t C, int64_t gs0, int64_t gs1)
{
    __shared__ uint16_t t[128][66];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c0 = blockIdx.x * 128;
    const int64_t l0 = (int64_t)blockIdx.y * 64;
    const int64_t n = blockIdx.z;
    const uint16_t *src = gy + n * gs0;
    const int64_t l = l0 + lane;
    // All 32 reads of a thread in flight before the first LDS write.
    uint16_t v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
        const int c = c0 + wv + 4 * u;
        v[u] = (c < C && l < L) ? src[(int64_t)c * gs1 + l] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) t[wv + 4 * u][lane] = v[u];
    __syncthreads();
    uint32_t *dst = reinterpret_cast<uint32_t *>(out + n * L * C);
    const int c = c0 + 2 * lane;
#pragma unroll
    for (int r = wv; r < 64; r += 4) {
        const int64_t lr = l0 + r;
        if (lr < L && c < C)
            dst[(lr * C + c) >> 1] = (uint32_t)t[2 * lane][r] | ((uint32_t)t[2 * lane + 1][r] << 16);
    }
}

int launch_gy_to_cl(const conv_bwd_plan_t &p, const void *gy, void *dst, void *stream)
{
    const conv_desc &d = p.d;
    if (esize(d.dtype) != 2 || p.gy.strides[1] == 1) return CONV_EINVAL;
    int64_t L = 1;
    for (int i = 0; i < d.spatial; ++i) L *= d.out[i];
    if (d.N == 0 || L == 0 || d.C_out == 0) return CONV_OK;
    if (d.N > 65535 || cdiv(L, 64) > 65535) return CONV_EUNSUPPORTED;
    if (d.C_out % 2 != 0) return CONV_EINVAL;
    hipLaunchKernelGGL(gy_to_cl_kernel, dim3((unsigned)cdiv(d.C_out, 128), (unsigned)cdiv(L, 64), (unsigned)d.N),
                       dim3(256), 0, static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(gy),
                       static_cast<uint16_t *>(dst), L, (int32_t)d.C_out, p.gy.strides[0], p.gy.strides[1]);
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

int launch_wgrad(const conv_bwd_plan_t &p, const void *x, const void *gy, void *dw, void *ws, void *stream)
{
    const conv_desc &d = p.d;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool tr = d.transposed != 0;
    // P: the operand dense over the positions m; Q: the gathered one.
    const conv_tensor &P = tr ? d.x : p.gy;
    const conv_tensor &Q = tr ? p.gy : d.x;
    WgArgs a;
    a.P = tr ? x : gy;
    a.Q = tr ? gy : x;
    a.part = static_cast<float *>(ws);
    a.ps_n = P.strides[0];
    a.ps_c = P.strides[1];
    a.qs_n = Q.strides[0];
    a.qs_c = Q.strides[1];
    // The used spatial dims are right-aligned in the three slots (unused
    // leading slots: extent 1, stride 0), so the fastest slot is the last
    // spatial dim of every rank -- the one a position-major chunk runs along.
    // The flat tap order (t0*K1 + t1)*K2 + t2 is unchanged by leading 1s.
    const int lead = 3 - d.spatial;
    for (int i = 0; i < 3; ++i) {
        const int j = i - lead;          // spatial dim held by slot i, or < 0
        const bool on = j >= 0;
        a.ps_l[i] = on ? P.strides[2 + j] : 0;
        a.qs_l[i] = on ? Q.strides[2 + j] : 0;
        a.E[i] = on ? (int32_t)(tr ? d.in[j] : d.out[j]) : 1;
        a.F[i] = on ? (int32_t)(tr ? d.out[j] : d.in[j]) : 1;
        a.K[i] = on ? (int32_t)d.k[j] : 1;
        a.S[i] = on ? (int32_t)d.stride[j] : 1;
        a.PB[i] = on ? (int32_t)d.padding_before[j] : 0;
        a.D[i] = on ? (int32_t)d.dilation[j] : 1;
    }
    a.N = (int32_t)d.N;
    a.G = (int32_t)d.groups;
    const int32_t Cig = (int32_t)(d.C_in / d.groups), Cog = (int32_t)(d.C_out / d.groups);
    a.PC = tr ? Cig : Cog;
    a.QC = tr ? Cog : Cig;
    a.T = (int32_t)(d.k[0] * d.k[1] * d.k[2]);
    a.apad = (int32_t)p.wg_tile[WB_APAD];
    a.bpad = (int32_t)p.wg_tile[WB_BPAD];
    a.splits = (int32_t)p.wg_tile[WB_SPLITS];
    a.M = (int64_t)d.N * a.E[0] * a.E[1] * a.E[2];
    a.p_bytes = (int32_t)p.wg_tile[WB_PBYTES];
    a.q_bytes = (int32_t)p.wg_tile[WB_QBYTES];
    a.PH2 = d.spatial == 2 ? (int32_t)d.padding_after[0] : 0;
    a.PW2 = (int32_t)d.padding_after[d.spatial - 1];
    if (p.wg_tile[WB_MFMA] == WB_PLANE) {
        const size_t lds = (size_t)wgrad_plane_lds(d);
        const dim3 blocks((unsigned)((int64_t)a.G * a.splits));
        switch (d.dtype) {
        case CONV_F32: hipLaunchKernelGGL((wgrad_plane_kernel<float>), blocks, dim3(256), lds, s, a); break;
        case CONV_F16: hipLaunchKernelGGL((wgrad_plane_kernel<f16_t>), blocks, dim3(256), lds, s, a); break;
        default: hipLaunchKernelGGL((wgrad_plane_kernel<bf16_t>), blocks, dim3(256), lds, s, a); break;
        }
        if (hipGetLastError() != hipSuccess) return CONV_EDEVICE;
    }
    const bool dwk = p.wg_tile[WB_MFMA] == WB_DW;
    const bool mfma = p.wg_tile[WB_MFMA] != 0 && !dwk && p.wg_tile[WB_MFMA] != WB_PLANE;
    const bool pm_p = (p.wg_tile[WB_MFMA] & 2) != 0, pm_q = (p.wg_tile[WB_MFMA] & 4) != 0;
    hipError_t e = hipSuccess;
    if (p.wg_tile[WB_MFMA] != WB_PLANE) {
        switch (d.dtype) {
        case CONV_F32: e = launch_wgrad_t<float>(a, false, false, false, s); break;
        case CONV_F16: e = dwk ? launch_wgrad_dw<f16_t>(a, s) : launch_wgrad_t<f16_t>(a, mfma, pm_p, pm_q, s); break;
        default: e = dwk ? launch_wgrad_dw<bf16_t>(a, s) : launch_wgrad_t<bf16_t>(a, mfma, pm_p, pm_q, s); break;
        }
    }
    if (e != hipSuccess) return CONV_EDEVICE;
    RdArgs r;
    r.part = a.part;
    r.out = dw;
    r.count = (int64_t)a.G * a.T * a.PC * a.QC;
    r.plane = (int64_t)a.G * a.T * a.apad * a.bpad;
    r.splits = a.splits;
    r.is_w = 1;
    r.G = a.G;
    r.T = a.T;
    r.PC = a.PC;
    r.QC = a.QC;
    r.apad = a.apad;
    r.bpad = a.bpad;
    r.K1 = a.K[1];
    r.K2 = a.K[2];
    r.os0 = p.dw.strides[0];
    r.os1 = p.dw.strides[1];
    for (int i = 0; i < 3; ++i) r.osk[i] = i >= lead ? p.dw.strides[2 + i - lead] : 0;   // the slots of a.K
    switch (d.dtype) {
    case CONV_F32: e = launch_reduce_t<float>(r, s); break;
    case CONV_F16: e = launch_reduce_t<f16_t>(r, s); break;
    default: e = launch_reduce_t<bf16_t>(r, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

int launch_bgrad(const conv_bwd_plan_t &p, const void *gy, void *db, void *ws, void *stream)
{
    const conv_desc &d = p.d;
    hipStream_t s = static_cast<hipStream_t>(stream);
    BgArgs b;
    b.gy = gy;
    b.part = static_cast<float *>(ws);
    b.gs_n = p.gy.strides[0];
    b.gs_c = p.gy.strides[1];
    for (int i = 0; i < 3; ++i) {
        b.gs_l[i] = i < d.spatial ? p.gy.strides[2 + i] : 0;
        b.O[i] = (int32_t)d.out[i];
    }
    b.N = (int32_t)d.N;
    b.C = (int32_t)d.C_out;
    b.splits = (int32_t)p.db_splits;
    b.M = (int64_t)d.N * b.O[0] * b.O[1] * b.O[2];
    const bool rows = bgrad_by_rows(d, p.gy);
    hipError_t e;
    switch (d.dtype) {
    case CONV_F32: e = launch_bgrad_t<float>(b, rows, s); break;
    case CONV_F16: e = launch_bgrad_t<f16_t>(b, rows, s); break;
    default: e = launch_bgrad_t<bf16_t>(b, rows, s); break;
    }
    if (e != hipSuccess) return CONV_EDEVICE;
    RdArgs r;
    std::memset(&r, 0, sizeof(r));
    r.part = b.part;
    r.out = db;
    r.count = b.C;
    r.plane = b.C;
    r.splits = b.splits;
    r.is_w = 0;
    r.os0 = p.db.rank > 0 ? p.db.strides[0] : 1;
    switch (d.dtype) {
    case CONV_F32: e = launch_reduce_t<float>(r, s); break;
    case CONV_F16: e = launch_reduce_t<f16_t>(r, s); break;
    default: e = launch_reduce_t<bf16_t>(r, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
