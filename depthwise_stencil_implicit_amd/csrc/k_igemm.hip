// Implicit-GEMM convolution for gfx950 (kernels CONV_K_IGEMM, CONV_K_IGEMM_T).
//
// The convolution is the GEMM  C[m, co] = sum_k A[m, k] * B[k, co]  with
//   m  = an output position (n, o_1..o_r) of one group,
//   co = an output channel of that group,
//   k  = (tap t, input channel c), tap-major so that one K step reads a run of
//        channels of one input pixel,
//   A[m, (t, c)] = x[n, g*Cig + c, input position of (m, t)], zero when absent,
//   B[(t, c), co] = the weight of (co, c, t).
// A is never materialised: each K step gathers its [BM x BK] tile straight from
// x into LDS (executorch PR #25091, "Run transposed convolutions on the
// implicit-GEMM template", description: pixel tiles, a tap-major K order, and
// one flag that switches the gather to the transposed index map; torch/
// _inductor/kernel/conv.py, conv2d_template: rows are output pixels, columns
// output channels, the group a separate launch axis).
//
// Forward gather (LOOP_BODY_2D in torch/_inductor/kernel/conv.py):
//     input = o*s - pb + t*dil, absent outside [0, L).
// Transposed gather (PR #25091 description, second paragraph):
//     input = (o + pb - t*dil) / s, present only for an exact in-range quotient.
// The transposed rows are split by output phase rho = o mod s (per dim).  For
// o = s*j + rho the quotient is  j + (rho + pb - t*dil)/s,  and it is exact for
// a tap t only when (rho + pb - t*dil) is divisible by s -- a property of the
// phase, not of the row.  So each workgroup serves one phase, runs its K loop
// over that phase's taps only, and is a plain stride-1 gather over j: the
// structurally-zero taps the literal gather would multiply are never visited.
//
// Weights are first repacked (into the caller's workspace) to
// [G][Cog_pad][taps][Cig_pad], zero-padded, so every B load is a 16-byte vector.
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}; fp32 inputs use eight
// v_mfma_f32_16x16x4_f32 steps per 32-wide K slice.  fp32 accumulation.
#include "dev_common.h"
#include "internal.h"

#include <algorithm>

namespace miconv {

struct IgArgs {
    const void *x;
    const void *w;  // repacked
    const void *b;
    void *y;
    int64_t xs_n, xs_c, xs_l[3];
    int64_t ys_n, ys_c, ys_l[3];
    int64_t rows;  // rows per phase: N * J0 * J1 * J2
    int32_t Cig, Cog, cig_pad, cog_pad, taps;
    int32_t L[3], K[3], O[3], S[3], PB[3], D[3], J[3];
    int32_t G, phases, m_tiles, n_tiles, transposed, has_bias;
    int32_t total_tiles;
};

// Block index -> tile index, so that each XCD (blocks are dealt to the 8 XCDs
// round-robin) receives one contiguous range of tiles: neighbouring tiles share
// halo rows and weight slices in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int total)
{
    const int q = total >> 3, r = total & 7;
    const int xcd = b & 7, local = b >> 3;
    const int off = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return off + local;
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void igemm_kernel(IgArgs a)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int ES = Dt<T>::size;
    constexpr int EV = 16 / ES;           // elements per 16-byte chunk
    constexpr int CH = BK / EV;           // chunks per tile row
    constexpr int LDK = BK + EV;          // LDS row pitch (elements), one chunk of skew
    constexpr int A_IT = (BM * CH + NT - 1) / NT;
    constexpr int B_IT = (BN * CH + NT - 1) / NT;
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert(NT % CH == 0, "chunk column must be fixed per thread");
    static_assert(BK % 32 == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (BM + BN) * LDK * ES];
    T *sA = reinterpret_cast<T *>(smem);
    T *sB = sA + 2 * BM * LDK;

    const int tid = threadIdx.x;
    const int tile = xcd_tile(blockIdx.x, a.total_tiles);
    const int n_tile = tile % a.n_tiles;
    int rest = tile / a.n_tiles;
    const int m_tile = rest % a.m_tiles;
    rest /= a.m_tiles;
    const int phase = rest % a.phases;
    const int g = rest / a.phases;

    // Phase residues (transposed); zero for forward calls.
    int rho[3];
    {
        int p = phase;
        rho[2] = p % a.S[2]; p /= a.S[2];
        rho[1] = p % a.S[1]; p /= a.S[1];
        rho[0] = p;
        if (!a.transposed) rho[0] = rho[1] = rho[2] = 0;
    }

    const T *__restrict__ X = static_cast<const T *>(a.x);
    const T *__restrict__ W = static_cast<const T *>(a.w);

    // ---- per-thread A rows (fixed for the whole K loop) ----
    const int kc = tid % CH;
    int64_t a_nb[A_IT];
    int a_base[A_IT][3];
    bool a_ok[A_IT];
    const int64_t JJ = (int64_t)a.J[0] * a.J[1] * a.J[2];
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
        const int row = (tid + i * NT) / CH;
        const int64_t m = (int64_t)m_tile * BM + row;
        bool ok = row < BM && m < a.rows;
        int64_t n = 0;
        int j[3] = {0, 0, 0};
        if (ok) {
            n = m / JJ;
            int64_t r = m - n * JJ;
            j[2] = (int)(r % a.J[2]);
            r /= a.J[2];
            j[1] = (int)(r % a.J[1]);
            j[0] = (int)(r / a.J[1]);
        }
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            if (a.transposed) {
                ok = ok && (a.S[d] * j[d] + rho[d] < a.O[d]);
                a_base[i][d] = j[d];
            } else {
                a_base[i][d] = j[d] * a.S[d] - a.PB[d];
            }
        }
        a_ok[i] = ok;
        a_nb[i] = n * a.xs_n + (int64_t)g * a.Cig * a.xs_c;
    }

    // Tap validity for this phase (uniform across the workgroup).
    auto tap_off = [&](int t, int off[3]) -> bool {
        int tt[3];
        tt[2] = t % a.K[2];
        tt[1] = (t / a.K[2]) % a.K[1];
        tt[0] = t / (a.K[2] * a.K[1]);
        bool ok = true;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            if (a.transposed) {
                const int num = rho[d] + a.PB[d] - tt[d] * a.D[d];
                const int md = num % a.S[d];
                ok = ok && (md == 0);
                off[d] = num / a.S[d];
            } else {
                off[d] = tt[d] * a.D[d];
            }
        }
        return ok;
    };
    auto next_tap = [&](int t, int off[3]) -> int {
        while (t < a.taps && !tap_off(t, off)) ++t;
        return t;
    };

    const int ncb = a.cig_pad / BK;

    uint4 ra[A_IT], rb[B_IT];
    auto gload = [&](int t, const int off[3], int cb) {
        const int c = cb * BK + kc * EV;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int i0 = a_base[i][0] + off[0], i1 = a_base[i][1] + off[1], i2 = a_base[i][2] + off[2];
            const bool inb = a_ok[i] && (unsigned)i0 < (unsigned)a.L[0] && (unsigned)i1 < (unsigned)a.L[1] &&
                             (unsigned)i2 < (unsigned)a.L[2];
            const int64_t pix = a_nb[i] + i0 * a.xs_l[0] + i1 * a.xs_l[1] + i2 * a.xs_l[2];
            if (VEC) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (inb && c < a.Cig) v = *reinterpret_cast<const uint4 *>(X + pix + c);
                ra[i] = v;
            } else {
                T tmp[EV];
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    T z;
                    __builtin_memset(&z, 0, sizeof(T));
                    tmp[e] = (inb && c + e < a.Cig) ? X[pix + (int64_t)(c + e) * a.xs_c] : z;
                }
                __builtin_memcpy(&ra[i], tmp, 16);
            }
        }
        const int64_t wrow0 = ((int64_t)g * a.cog_pad + (int64_t)n_tile * BN) * a.taps;
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
            const int col = (tid + i * NT) / CH;
            if (col < BN) {
                const int64_t off_w = ((wrow0 + (int64_t)col * a.taps + t) * a.cig_pad) + cb * BK + kc * EV;
                rb[i] = *reinterpret_cast<const uint4 *>(W + off_w);
            }
        }
    };
    auto sstore = [&](int stage) {
        T *A = sA + stage * BM * LDK;
        T *B = sB + stage * BN * LDK;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int row = (tid + i * NT) / CH;
            if (row < BM) *reinterpret_cast<uint4 *>(A + row * LDK + kc * EV) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
            const int col = (tid + i * NT) / CH;
            if (col < BN) *reinterpret_cast<uint4 *>(B + col * LDK + kc * EV) = rb[i];
        }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wr = wave / WN, wc = wave % WN;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage) {
        const T *A = sA + stage * BM * LDK;
        const T *B = sB + stage * BN * LDK;
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int koff = kk * 32 + (lane >> 4) * 8;
            if constexpr (ES == 2) {
                uint4 af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = *reinterpret_cast<const uint4 *>(A + (wr * TM + i * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[j] = *reinterpret_cast<const uint4 *>(B + (wc * TN + j * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) mma_16x16x32(af[i], bfr[j], acc[i][j], T{});
            } else {
                float af[FM][8], bfr[FN][8];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const float *p = reinterpret_cast<const float *>(A) + (wr * TM + i * 16 + (lane & 15)) * LDK + koff;
                    const float4 v0 = *reinterpret_cast<const float4 *>(p);
                    const float4 v1 = *reinterpret_cast<const float4 *>(p + 4);
                    af[i][0] = v0.x; af[i][1] = v0.y; af[i][2] = v0.z; af[i][3] = v0.w;
                    af[i][4] = v1.x; af[i][5] = v1.y; af[i][6] = v1.z; af[i][7] = v1.w;
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const float *p = reinterpret_cast<const float *>(B) + (wc * TN + j * 16 + (lane & 15)) * LDK + koff;
                    const float4 v0 = *reinterpret_cast<const float4 *>(p);
                    const float4 v1 = *reinterpret_cast<const float4 *>(p + 4);
                    bfr[j][0] = v0.x; bfr[j][1] = v0.y; bfr[j][2] = v0.z; bfr[j][3] = v0.w;
                    bfr[j][4] = v1.x; bfr[j][5] = v1.y; bfr[j][6] = v1.z; bfr[j][7] = v1.w;
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) mma_16x16x32_f32(af[i], bfr[j], acc[i][j]);
            }
        }
    };

    // ---- K loop: (valid tap, channel block) steps, double-buffered LDS ----
    int off[3];
    int t = next_tap(0, off);
    int cb = 0;
    if (t < a.taps && ncb > 0) {
        gload(t, off, cb);
        sstore(0);
        __syncthreads();
        int stage = 0;
        while (true) {
            int nt = t, ncb_i = cb + 1;
            int noff[3] = {off[0], off[1], off[2]};
            if (ncb_i == ncb) {
                ncb_i = 0;
                nt = next_tap(t + 1, noff);
            }
            const bool more = nt < a.taps;
            if (more) gload(nt, noff, ncb_i);
            compute(stage);
            if (more) sstore(stage ^ 1);
            __syncthreads();
            if (!more) break;
            stage ^= 1;
            t = nt;
            cb = ncb_i;
            off[0] = noff[0]; off[1] = noff[1]; off[2] = noff[2];
        }
    }

    // ---- epilogue: bias in fp32, one rounding, store at y's strides ----
    T *__restrict__ Y = static_cast<T *>(a.y);
    const T *__restrict__ Bias = static_cast<const T *>(a.b);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int co = n_tile * BN + wc * TN + j * 16 + (lane & 15);
        if (co >= a.Cog) continue;
        const int cog = g * a.Cog + co;
        const float bias = a.has_bias ? to_f32(Bias[cog]) : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = wr * TM + i * 16 + (lane >> 4) * 4 + e;
                const int64_t m = (int64_t)m_tile * BM + row;
                if (m >= a.rows) continue;
                const int64_t n = m / JJ;
                int64_t r = m - n * JJ;
                int o[3];
                o[2] = (int)(r % a.J[2]);
                r /= a.J[2];
                o[1] = (int)(r % a.J[1]);
                o[0] = (int)(r / a.J[1]);
                bool ok = true;
                if (a.transposed) {
#pragma unroll
                    for (int d = 0; d < 3; ++d) {
                        o[d] = a.S[d] * o[d] + rho[d];
                        ok = ok && o[d] < a.O[d];
                    }
                }
                if (!ok) continue;
                const int64_t yo = n * a.ys_n + (int64_t)cog * a.ys_c + o[0] * a.ys_l[0] + o[1] * a.ys_l[1] +
                                   o[2] * a.ys_l[2];
                Y[yo] = from_f32<T>(acc[i][j][e] + bias);
            }
        }
    }
}

// Weight repack: w (any strides) -> [G][Cog_pad][taps][Cig_pad], zero padded.
template <typename T>
__global__ void igemm_repack(const T *__restrict__ w, T *__restrict__ wr, int64_t total, int32_t Cig, int32_t Cog,
                             int32_t cig_pad, int32_t cog_pad, int32_t taps, int32_t K1, int32_t K2, int64_t ws0,
                             int64_t ws1, int64_t wk0, int64_t wk1, int64_t wk2, int32_t transposed)
{
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % cig_pad);
        int64_t r = idx / cig_pad;
        const int t = (int)(r % taps);
        r /= taps;
        const int j = (int)(r % cog_pad);
        const int64_t g = r / cog_pad;
        T v;
        __builtin_memset(&v, 0, sizeof(T));
        if (j < Cog && c < Cig) {
            const int t2 = t % K2, t1 = (t / K2) % K1, t0 = t / (K2 * K1);
            const int64_t toff = t0 * wk0 + t1 * wk1 + t2 * wk2;
            if (!transposed)
                v = w[(g * Cog + j) * ws0 + (int64_t)c * ws1 + toff];
            else
                v = w[(g * Cig + c) * ws0 + (int64_t)j * ws1 + toff];
        }
        wr[idx] = v;
    }
}

namespace {

constexpr IgemmCfg kCfgs[] = {
    {128, 128, 32, 2, 2},  // 0: 2-byte types, wide N
    {128, 64, 32, 2, 2},   // 1: 2-byte types, N <= 64
    {256, 32, 32, 4, 1},   // 2: 2-byte types, N <= 32
    {64, 64, 32, 2, 2},    // 3: fp32
};

template <typename T, int V, bool VEC>
hipError_t launch_cfg(const IgArgs &a, hipStream_t s)
{
    constexpr IgemmCfg c = kCfgs[V];
    hipLaunchKernelGGL((igemm_kernel<T, c.bm, c.bn, c.bk, c.wm, c.wn, VEC>), dim3(a.total_tiles),
                       dim3(64 * c.wm * c.wn), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const IgArgs &a, int variant, bool vec, hipStream_t s)
{
    if constexpr (Dt<T>::size == 4) {
        return vec ? launch_cfg<T, 3, true>(a, s) : launch_cfg<T, 3, false>(a, s);
    } else {
        switch (variant) {
        case 0: return vec ? launch_cfg<T, 0, true>(a, s) : launch_cfg<T, 0, false>(a, s);
        case 1: return vec ? launch_cfg<T, 1, true>(a, s) : launch_cfg<T, 1, false>(a, s);
        case 2: return vec ? launch_cfg<T, 2, true>(a, s) : launch_cfg<T, 2, false>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
}

template <typename T>
hipError_t launch_repack(const conv_plan_t &p, const void *w, void *ws, hipStream_t s)
{
    const conv_desc &d = p.d;
    const int64_t taps = d.k[0] * d.k[1] * d.k[2];
    const int64_t total = d.groups * p.tile[IG_COG_PAD] * taps * p.tile[IG_CIG_PAD];
    if (total == 0) return hipSuccess;
    const int r = d.spatial;
    int64_t wk[3] = {0, 0, 0};
    for (int i = 0; i < r; ++i) wk[i] = d.w.strides[2 + i];
    const int64_t blocks = std::min<int64_t>(cdiv(total, 256), 4096);
    hipLaunchKernelGGL((igemm_repack<T>), dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const T *>(w),
                       static_cast<T *>(ws), total, (int32_t)(d.C_in / d.groups), (int32_t)(d.C_out / d.groups),
                       (int32_t)p.tile[IG_CIG_PAD], (int32_t)p.tile[IG_COG_PAD], (int32_t)taps, (int32_t)d.k[1],
                       (int32_t)d.k[2], d.w.strides[0], d.w.strides[1], wk[0], wk[1], wk[2], d.transposed);
    return hipGetLastError();
}

}  // namespace

const IgemmCfg &igemm_cfg(int variant) { return kCfgs[variant]; }
int igemm_num_cfgs() { return (int)(sizeof(kCfgs) / sizeof(kCfgs[0])); }

int launch_igemm(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *ws,
                 void *stream, bool vec)
{
    const conv_desc &d = p.d;
    hipStream_t s = static_cast<hipStream_t>(stream);
    IgArgs a;
    a.x = x;
    a.w = ws;
    a.b = b;
    a.y = y;
    const int r = d.spatial;
    a.xs_n = d.x.strides[0];
    a.xs_c = d.x.strides[1];
    a.ys_n = p.y.strides[0];
    a.ys_c = p.y.strides[1];
    for (int i = 0; i < 3; ++i) {
        const bool on = i < r;
        a.xs_l[i] = on ? d.x.strides[2 + i] : 0;
        a.ys_l[i] = on ? p.y.strides[2 + i] : 0;
        a.L[i] = (int32_t)d.in[i];
        a.K[i] = (int32_t)d.k[i];
        a.O[i] = (int32_t)d.out[i];
        a.S[i] = (int32_t)d.stride[i];
        a.PB[i] = (int32_t)d.padding_before[i];
        a.D[i] = (int32_t)d.dilation[i];
        a.J[i] = (int32_t)(d.transposed ? cdiv(d.out[i], d.stride[i]) : d.out[i]);
    }
    a.Cig = (int32_t)(d.C_in / d.groups);
    a.Cog = (int32_t)(d.C_out / d.groups);
    a.cig_pad = (int32_t)p.tile[IG_CIG_PAD];
    a.cog_pad = (int32_t)p.tile[IG_COG_PAD];
    a.taps = (int32_t)(d.k[0] * d.k[1] * d.k[2]);
    a.G = (int32_t)d.groups;
    a.phases = (int32_t)p.tile[IG_PHASES];
    a.m_tiles = (int32_t)p.tile[IG_MTILES];
    a.n_tiles = (int32_t)p.tile[IG_NTILES];
    a.rows = p.tile[IG_ROWS];
    a.transposed = d.transposed;
    a.has_bias = d.has_bias;
    a.total_tiles = (int32_t)p.grid[0];

    hipError_t e;
    switch (d.dtype) {
    case CONV_F32: e = launch_repack<float>(p, w, ws, s); break;
    case CONV_F16: e = launch_repack<f16_t>(p, w, ws, s); break;
    default: e = launch_repack<bf16_t>(p, w, ws, s); break;
    }
    if (e != hipSuccess) return CONV_EDEVICE;
    switch (d.dtype) {
    case CONV_F32: e = launch_typed<float>(a, p.variant, vec, s); break;
    case CONV_F16: e = launch_typed<f16_t>(a, p.variant, vec, s); break;
    default: e = launch_typed<bf16_t>(a, p.variant, vec, s); break;
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
