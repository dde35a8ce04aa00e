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
// gfx950 mapping
//   * Weights are first repacked (into the caller's workspace) to
//     [G][Cog_pad][taps][Cig_pad], zero padded, so B tiles are 16-byte loads.
//   * A rows are gathered with raw buffer loads: an absent input position gets
//     an out-of-range offset and the hardware returns zeros, so padding costs
//     no branch and a thread's loads of one K step are all in flight together.
//   * LDS tiles hold rows of 8 sixteen-byte chunks; chunk c of row r is stored
//     at position c ^ (r & 7), so the 8 lanes that share a read cycle hit 8
//     different bank groups.  Two stages: the next step's global loads are in
//     flight while the MFMAs consume the current stage.
//   * MFMA v_mfma_f32_16x16x32_{bf16,f16} (fp32: eight v_mfma_f32_16x16x4_f32
//     per 32-wide K slice) with operands swapped -- weights as the MFMA A
//     operand -- so each lane ends holding 4 consecutive output channels of one
//     output position: one 8-byte store per lane into channel-contiguous y.
//   * Workgroups are dealt to the 8 XCDs round-robin; the block index is
//     remapped so each XCD gets one contiguous range of tiles (shared halo
//     rows and weight slices stay in that XCD's L2).
#include "dev_common.h"
#include "internal.h"

#include <algorithm>
#include <type_traits>

namespace miconv {

struct IgArgs {
    const void *x;
    const void *w;  // repacked weights
    const void *b;
    void *y;
    int64_t ys_n, ys_c, ys_l[3];
    int32_t xs_n, xs_c, xs_l[3];  // element strides of x (32-bit: the planner keeps the span < 2 GB)
    int32_t x_bytes;
    int32_t rows;                 // rows per phase: N * J0 * J1 * J2
    int32_t Cig, Cog, cig_pad, cog_pad, taps;
    int32_t L[3], K[3], O[3], S[3], PB[3], D[3], J[3];
    int32_t G, phases, m_tiles, n_tiles, transposed, has_bias;
    int32_t total_tiles, y_vec4;
    int32_t row0;                 // first row (of every phase) this launch covers
    int32_t ksplit;               // K ranges per tile (> 1: fp32 partial sums into part)
    float *part;                  // [ksplit][G][phases][rows - row0][cog_pad] partial sums
    int32_t w_bytes;              // bytes of the repacked weights (buffer range)
    int32_t one;                  // 1x1 plain GEMM: row m of A is x's row m (m * Cig elements)
    int32_t y_lin;                // 16-bit forward output whose row m starts at element m * y_rs (+ channel)
    int32_t y_rs;
};

// Byte offset of 16-byte chunk `c` of LDS row `r` (rows of 8 chunks).
__device__ __forceinline__ int swz(int r, int c) { return (r * 8 + (c ^ (r & 7))) * 16; }

template <typename T, int BM, int BN, int WM, int WN, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void igemm_kernel(IgArgs a)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int ES = Dt<T>::size;
    constexpr int EV = 16 / ES;            // elements per chunk
    constexpr int BK = 8 * EV;             // K elements per step (8 chunks per row)
    constexpr int A_IT = BM * 8 / NT;      // A chunks per thread per step
    constexpr int B_IT = BN * 8 / NT;      // B chunks per thread per step
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0 && NT % 8 == 0, "chunks per thread");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *sA = smem;                        // [2][BM][8 chunks]
    unsigned char *sB = smem + 2 * BM * 128;         // [2][BN][8 chunks]

    const int tid = threadIdx.x;
    const int tile = xcd_tile(blockIdx.x, a.total_tiles);
    // Tile order (fastest first): column tile, phase, row tile, group -- the
    // tiles that gather the same input rows run side by side on one XCD.
    const int n_tile = tile % a.n_tiles;
    int rest = tile / a.n_tiles;
    const int phase = rest % a.phases;
    rest /= a.phases;
    const int m_tile = rest % a.m_tiles;
    const int g = rest / a.m_tiles;

    int rho0 = 0, rho1 = 0, rho2 = 0;
    if (a.transposed) {
        int p = phase;
        rho2 = p % a.S[2];
        p /= a.S[2];
        rho1 = p % a.S[1];
        rho0 = p / a.S[1];
    }
    const int JJ = a.J[0] * a.J[1] * a.J[2];
    const int J12 = a.J[1] * a.J[2];

    // ---- A rows of this thread (fixed over the K loop) ----
    const int kc = tid & 7;
    int a_nb[A_IT], a_b0[A_IT], a_b1[A_IT], a_b2[A_IT];
    bool a_ok[A_IT];
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
        const int row = (tid >> 3) + i * (NT / 8);
        const int m = a.row0 + m_tile * BM + row;
        bool ok = m < a.rows;
        const int mm = ok ? m : 0;
        const int n = mm / JJ;
        const int r = mm - n * JJ;
        const int j0 = r / J12, r2 = r - j0 * J12;
        const int j1 = r2 / a.J[2], j2 = r2 - j1 * a.J[2];
        if (a.transposed) {
            ok = ok && a.S[0] * j0 + rho0 < a.O[0] && a.S[1] * j1 + rho1 < a.O[1] && a.S[2] * j2 + rho2 < a.O[2];
            a_b0[i] = j0;
            a_b1[i] = j1;
            a_b2[i] = j2;
        } else {
            a_b0[i] = j0 * a.S[0] - a.PB[0];
            a_b1[i] = j1 * a.S[1] - a.PB[1];
            a_b2[i] = j2 * a.S[2] - a.PB[2];
        }
        a_ok[i] = ok;
        a_nb[i] = n * a.xs_n + g * a.Cig * a.xs_c;
    }

    // Tap t -> input offsets for this phase; false when the tap is absent.
    auto tap_offsets = [&](int t, int &o0, int &o1, int &o2) -> bool {
        const int t2 = t % a.K[2];
        const int t01 = t / a.K[2];
        const int t1 = t01 % a.K[1];
        const int t0 = t01 / a.K[1];
        if (!a.transposed) {
            o0 = t0 * a.D[0];
            o1 = t1 * a.D[1];
            o2 = t2 * a.D[2];
            return true;
        }
        const int n0 = rho0 + a.PB[0] - t0 * a.D[0];
        const int n1 = rho1 + a.PB[1] - t1 * a.D[1];
        const int n2 = rho2 + a.PB[2] - t2 * a.D[2];
        o0 = n0 / a.S[0];
        o1 = n1 / a.S[1];
        o2 = n2 / a.S[2];
        return n0 % a.S[0] == 0 && n1 % a.S[1] == 0 && n2 % a.S[2] == 0;
    };

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.w), (short)0, a.w_bytes, 0x00020000);
    const T *__restrict__ X = static_cast<const T *>(a.x);
    const int ncb = a.cig_pad / BK;
    // B chunk offsets: per-thread constant part; the step adds a uniform part.
    const int wtile0 = (g * a.cog_pad + n_tile * BN) * a.taps * a.cig_pad * ES;
    int b_off[B_IT];
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
        const int col = (tid >> 3) + i * (NT / 8);
        b_off[i] = (col * a.taps * a.cig_pad + kc * EV) * ES;
    }

    uint4 ra[A_IT], rb[B_IT];
    auto gload = [&](int t, int o0, int o1, int o2, int cb) {
        const int c = cb * BK + kc * EV;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int i0 = a_b0[i] + o0, i1 = a_b1[i] + o1, i2 = a_b2[i] + o2;
            const bool inb = a_ok[i] && (unsigned)i0 < (unsigned)a.L[0] && (unsigned)i1 < (unsigned)a.L[1] &&
                             (unsigned)i2 < (unsigned)a.L[2];
            const int pix = a_nb[i] + i0 * a.xs_l[0] + i1 * a.xs_l[1] + i2 * a.xs_l[2];
            if constexpr (VEC) {
                const int off = (inb && c < a.Cig) ? (pix + c) * ES : 0x7fffffff;
                ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            } else {
                T tmp[EV];
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const bool ok = inb && c + e < a.Cig;
                    const int idx = ok ? pix + (c + e) * a.xs_c : 0;
                    T v = X[idx];
                    if (!ok) __builtin_memset(&v, 0, sizeof(T));
                    tmp[e] = v;
                }
                __builtin_memcpy(&ra[i], tmp, 16);
            }
        }
        const int step_off = wtile0 + (t * a.cig_pad + cb * BK) * ES;
#pragma unroll
        for (int i = 0; i < B_IT; ++i)
            rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, b_off[i], step_off, 0));
    };
    auto sstore = [&](int stage) {
        unsigned char *A = sA + stage * BM * 128;
        unsigned char *B = sB + stage * BN * 128;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int row = (tid >> 3) + i * (NT / 8);
            *reinterpret_cast<uint4 *>(A + swz(row, kc)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
            const int col = (tid >> 3) + i * (NT / 8);
            *reinterpret_cast<uint4 *>(B + swz(col, kc)) = rb[i];
        }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wr = wave / WN, wc = wave % WN;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage) {
        const unsigned char *A = sA + stage * BM * 128;
        const unsigned char *B = sB + stage * BN * 128;
        if constexpr (ES == 2) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 af[FM], bf[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wr * TM + i * 16 + lr;
                    af[i] = *reinterpret_cast<const uint4 *>(A + swz(r, kk * 4 + lg));
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int r = wc * TN + j * 16 + lr;
                    bf[j] = *reinterpret_cast<const uint4 *>(B + swz(r, kk * 4 + lg));
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) mma_16x16x32(bf[j], af[i], acc[i][j], T{});
            }
        } else {
            float af[FM][8], bf[FN][8];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wr * TM + i * 16 + lr;
                const float4 v0 = *reinterpret_cast<const float4 *>(A + swz(r, 2 * lg));
                const float4 v1 = *reinterpret_cast<const float4 *>(A + swz(r, 2 * lg + 1));
                af[i][0] = v0.x; af[i][1] = v0.y; af[i][2] = v0.z; af[i][3] = v0.w;
                af[i][4] = v1.x; af[i][5] = v1.y; af[i][6] = v1.z; af[i][7] = v1.w;
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wc * TN + j * 16 + lr;
                const float4 v0 = *reinterpret_cast<const float4 *>(B + swz(r, 2 * lg));
                const float4 v1 = *reinterpret_cast<const float4 *>(B + swz(r, 2 * lg + 1));
                bf[j][0] = v0.x; bf[j][1] = v0.y; bf[j][2] = v0.z; bf[j][3] = v0.w;
                bf[j][4] = v1.x; bf[j][5] = v1.y; bf[j][6] = v1.z; bf[j][7] = v1.w;
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) mma_16x16x32_f32(bf[j], af[i], acc[i][j]);
        }
    };

    // ---- K loop over (valid tap, channel block), double-buffered ----
    int t = 0, o0 = 0, o1 = 0, o2 = 0;
    while (t < a.taps && !tap_offsets(t, o0, o1, o2)) ++t;
    if (t < a.taps && ncb > 0) {
        int cb = 0;
        gload(t, o0, o1, o2, cb);
        sstore(0);
        __syncthreads();
        int stage = 0;
        while (true) {
            int nt = t, ncbi = cb + 1, p0 = o0, p1 = o1, p2 = o2;
            if (ncbi == ncb) {
                ncbi = 0;
                ++nt;
                while (nt < a.taps && !tap_offsets(nt, p0, p1, p2)) ++nt;
            }
            const bool more = nt < a.taps;
            if (more) gload(nt, p0, p1, p2, ncbi);
            compute(stage);
            if (more) sstore(stage ^ 1);
            __syncthreads();
            if (!more) break;
            stage ^= 1;
            t = nt;
            cb = ncbi;
            o0 = p0;
            o1 = p1;
            o2 = p2;
        }
    }

    // ---- epilogue: lane holds 4 consecutive channels of one output position ----
    T *__restrict__ Y = static_cast<T *>(a.y);
    const T *__restrict__ Bias = static_cast<const T *>(a.b);
    float bias[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int co = n_tile * BN + wc * TN + j * 16 + lg * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            bias[j][e] = (a.has_bias && co + e < a.Cog) ? to_f32(Bias[g * a.Cog + co + e]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = a.row0 + m_tile * BM + wr * TM + i * 16 + lr;
        if (m >= a.rows) continue;
        const int n = m / JJ;
        const int r = m - n * JJ;
        int q0 = r / J12;
        const int r2 = r - q0 * J12;
        int q1 = r2 / a.J[2], q2 = r2 - q1 * a.J[2];
        if (a.transposed) {
            q0 = a.S[0] * q0 + rho0;
            q1 = a.S[1] * q1 + rho1;
            q2 = a.S[2] * q2 + rho2;
            if (q0 >= a.O[0] || q1 >= a.O[1] || q2 >= a.O[2]) continue;
        }
        const int64_t yrow = (int64_t)n * a.ys_n + q0 * a.ys_l[0] + q1 * a.ys_l[1] + q2 * a.ys_l[2];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int co = n_tile * BN + wc * TN + j * 16 + lg * 4;
            const int cg = g * a.Cog + co;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e] + bias[j][e];
            T *dst = Y + yrow + (int64_t)cg * a.ys_c;
            if (a.y_vec4) {
                // Cog % 4 == 0 here, so a group of 4 is either all in or all out.
                if (co < a.Cog) {
                    if constexpr (ES == 2) {
                        uint2 u;
                        u.x = pack2<T>(v[0], v[1]);
                        u.y = pack2<T>(v[2], v[3]);
                        *reinterpret_cast<uint2 *>(dst) = u;
                    } else {
                        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (co + e < a.Cog) dst[(int64_t)e * a.ys_c] = from_f32<T>(v[e]);
            }
        }
    }
}

// Vector path with direct-to-LDS loads.  Each buffer_load ... lds deposits one
// wave's 64 sixteen-byte chunks contiguously at a wave-uniform LDS address, so
// lane L of a wave covering rows r0..r0+7 fills slot (r0 + L/8, L%8) and
// fetches the logical chunk that the XOR swizzle puts there, (L%8) ^ (L/8).
// No registers hold tiles in flight, which leaves room for STAGES LDS stages:
// the loads of step s + STAGES - 1 are issued while step s is multiplied.
// An out-of-range offset deposits zeros, which is the padding.
//
// Each stage is its own LDS array and the step loop is unrolled by STAGES, so
// every stage is a compile-time choice: the compiler then only waits, before
// reading a stage, for the loads that target that stage.  The workgroup
// barrier is a bare s_barrier (a compiler-only memory clobber keeps LDS
// accesses on their side of it); before it each wave waits for its own loads of
// the stage about to be read, so after it every wave's loads have landed.  A
// fenced __syncthreads() would instead drain every load in flight.
// Launch bounds: a configuration whose stages fit in half the LDS (80 KB)
// runs two workgroups per CU, so its waves are held to the registers of
// twice as many waves per SIMD.
template <typename T, int BM, int BN, int WM, int WN, int STAGES, int KC>
__global__ __launch_bounds__(64 * WM * WN, (STAGES * (BM + BN) * KC * 16 <= 80 * 1024 ? 2 : 1) * WM * WN / 4) void
igemm_dma_kernel(IgArgs a)
{
    // The body uses LDS address-space pointers that only the device pass can
    // instantiate; the host pass needs nothing but the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NW = WM * WN;
    constexpr int ES = Dt<T>::size;
    constexpr int EV = 16 / ES;
    constexpr int BK = KC * EV;           // K elements per step
    constexpr int RPI = 64 / KC;          // rows one wave DMA instruction fills
    constexpr int RB = KC * 16;           // bytes per LDS row
    constexpr int A_IT = BM / (NW * RPI); // DMA instructions per wave per step, A tile
    constexpr int B_IT = BN / (NW * RPI);
    constexpr int LPS = A_IT + B_IT;      // loads per wave per step
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int STAGE_BYTES = (BM + BN) * RB;
    static_assert(KC == 4 || KC == 8, "chunks per row");
    static_assert(BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "rows per DMA round");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
    static_assert(STAGES >= 2 && STAGES <= 4 && (STAGES - 2) * LPS < 64, "stages / vmcnt range");

    __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st2[STAGES > 2 ? STAGE_BYTES : 16];
    __shared__ __attribute__((aligned(16))) unsigned char st3[STAGES > 3 ? STAGE_BYTES : 16];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int tile_k = xcd_tile(blockIdx.x, a.total_tiles);
    // Tile order (fastest first): K range, column tile, phase, row tile, group.
    const int ks = tile_k % a.ksplit;
    const int tile = tile_k / a.ksplit;
    const int n_tile = tile % a.n_tiles;
    int rest = tile / a.n_tiles;
    const int phase = rest % a.phases;
    rest /= a.phases;
    const int m_tile = rest % a.m_tiles;
    const int g = rest / a.m_tiles;

    int rho0 = 0, rho1 = 0, rho2 = 0;
    if (a.transposed) {
        int p = phase;
        rho2 = p % a.S[2];
        p /= a.S[2];
        rho1 = p % a.S[1];
        rho0 = p / a.S[1];
    }
    const int JJ = a.J[0] * a.J[1] * a.J[2];
    const int J12 = a.J[1] * a.J[2];

    // Rows this lane fetches: r = i*NW*RPI + wave*RPI + lane/KC, all with the
    // same row bits the swizzle uses, so the logical chunk kc is fixed.
    const int kc = KC == 8 ? ((lane & 7) ^ (lane >> 3)) : ((lane & 3) ^ ((lane >> 3) & 3));
    int a_nb[A_IT], a_b0[A_IT], a_b1[A_IT], a_b2[A_IT];
    bool a_ok[A_IT];
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
        const int row = i * NW * RPI + wave * RPI + lane / KC;
        const int m = a.row0 + m_tile * BM + row;
        bool ok = m < a.rows;
        const int mm = ok ? m : 0;
        const int n = mm / JJ;
        const int r = mm - n * JJ;
        const int j0 = r / J12, r2 = r - j0 * J12;
        const int j1 = r2 / a.J[2], j2 = r2 - j1 * a.J[2];
        if (a.transposed) {
            ok = ok && a.S[0] * j0 + rho0 < a.O[0] && a.S[1] * j1 + rho1 < a.O[1] && a.S[2] * j2 + rho2 < a.O[2];
            a_b0[i] = j0;
            a_b1[i] = j1;
            a_b2[i] = j2;
        } else {
            a_b0[i] = j0 * a.S[0] - a.PB[0];
            a_b1[i] = j1 * a.S[1] - a.PB[1];
            a_b2[i] = j2 * a.S[2] - a.PB[2];
        }
        a_ok[i] = ok;
        a_nb[i] = n * a.xs_n + g * a.Cig * a.xs_c;
    }
    const int wtile0 = (g * a.cog_pad + n_tile * BN) * a.taps * a.cig_pad * ES;
    int b_off[B_IT];
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
        const int col = i * NW * RPI + wave * RPI + lane / KC;
        b_off[i] = (col * a.taps * a.cig_pad + kc * EV) * ES;
    }

    auto tap_offsets = [&](int t, int &o0, int &o1, int &o2) -> bool {
        const int t2 = t % a.K[2];
        const int t01 = t / a.K[2];
        const int t1 = t01 % a.K[1];
        const int t0 = t01 / a.K[1];
        if (!a.transposed) {
            o0 = t0 * a.D[0];
            o1 = t1 * a.D[1];
            o2 = t2 * a.D[2];
            return true;
        }
        const int n0 = rho0 + a.PB[0] - t0 * a.D[0];
        const int n1 = rho1 + a.PB[1] - t1 * a.D[1];
        const int n2 = rho2 + a.PB[2] - t2 * a.D[2];
        o0 = n0 / a.S[0];
        o1 = n1 / a.S[1];
        o2 = n2 / a.S[2];
        return n0 % a.S[0] == 0 && n1 % a.S[1] == 0 && n2 % a.S[2] == 0;
    };

    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.w), (short)0, a.w_bytes, 0x00020000);
    typedef __attribute__((address_space(3))) void *lds_ptr;

    // Step cursor: (tap, channel block) over the phase's taps.
    const int ncb = a.cig_pad / BK;
    int it_t = 0, it_cb = 0, it_o0 = 0, it_o1 = 0, it_o2 = 0;
    while (it_t < a.taps && !tap_offsets(it_t, it_o0, it_o1, it_o2)) ++it_t;
    // Number of steps: valid taps x channel blocks (uniform); this workgroup
    // runs steps [kb, kb + nsteps) of them (its K range).
    int nall = 0;
    if (ncb > 0) {
        int dummy0, dummy1, dummy2;
        for (int t = 0; t < a.taps; ++t) nall += tap_offsets(t, dummy0, dummy1, dummy2) ? ncb : 0;
    }
    const int kb = ks * nall / a.ksplit;
    const int nsteps = (ks + 1) * nall / a.ksplit - kb;
    // Byte offsets of this lane's A rows at the current tap (channel chunk
    // kc of channel block 0), or the out-of-range marker for an absent
    // input position: recomputed only when the tap changes.  The channel
    // block rides in the scalar offset; the marker exceeds the buffer range
    // with any scalar offset added.
    int a_off[A_IT];
    auto set_tap = [&]() {
        if (a.one) {
            // 1x1: A is x's dense [rows, Cig] matrix.
#pragma unroll
            for (int i = 0; i < A_IT; ++i) {
                const int m = a.row0 + m_tile * BM + i * NW * RPI + wave * RPI + lane / KC;
                a_off[i] = m < a.rows ? (m * a.Cig + kc * EV) * ES : 0x7fffff00;
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int i0 = a_b0[i] + it_o0, i1 = a_b1[i] + it_o1, i2 = a_b2[i] + it_o2;
            const bool inb = a_ok[i] && (unsigned)i0 < (unsigned)a.L[0] && (unsigned)i1 < (unsigned)a.L[1] &&
                             (unsigned)i2 < (unsigned)a.L[2];
            const int pix = a_nb[i] + i0 * a.xs_l[0] + i1 * a.xs_l[1] + i2 * a.xs_l[2];
            a_off[i] = inb ? (pix + kc * EV) * ES : 0x7fffff00;
        }
    };
    auto advance = [&]() {
        if (++it_cb == ncb) {
            it_cb = 0;
            ++it_t;
            while (it_t < a.taps && !tap_offsets(it_t, it_o0, it_o1, it_o2)) ++it_t;
            set_tap();
        }
    };
    set_tap();
    for (int k = 0; k < kb; ++k) advance();
    // Channel chunks past Cig (a padded last block) read zeros.
    const bool cig_full = a.Cig % BK == 0;

    // Loads of the next step into stage A.  A dead issue (past the last
    // step) loads out of range everywhere, which fills the stage with zeros;
    // the cursor then runs past the last tap, harmlessly, so that the loads
    // stay on one path.
    auto issue = [&](unsigned char *A, bool live) {
        unsigned char *B = A + BM * RB;
        const int c = it_cb * BK + kc * EV;
        const bool cok = live && (cig_full || c < a.Cig);
#pragma unroll
        for (int i = 0; i < A_IT; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(A + (i * NW * RPI + wave * RPI) * RB), 16,
                                                     cok ? a_off[i] : 0x7fffff00, it_cb * BK * ES, 0, 0);
        const int step_off = wtile0 + (it_t * a.cig_pad + it_cb * BK) * ES;
#pragma unroll
        for (int i = 0; i < B_IT; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(B + (i * NW * RPI + wave * RPI) * RB), 16,
                                                     live ? b_off[i] : 0x7fffff00, step_off, 0, 0);
        advance();
    };

    const int wr = wave / WN, wc = wave % WN;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragment reads interleaved with the MFMAs, as one stream over the
    // step's K slices: the first slice's B fragments and first two A
    // fragments are read up front, then each group of FN MFMAs (one A
    // fragment) is followed by the read of the A fragment two groups ahead --
    // and, two groups before a slice starts, by that slice's B fragments --
    // so every read has two MFMA groups to land.  The scheduling groups pin
    // that order (the compiler's own schedule reads one A fragment and waits
    // for it before every group).  The refill of the stage read one step ago
    // is issued after the first slice's MFMAs.
    constexpr int KSL = KC / 4;                 // K slices (of 32) per step
    // This lane's fragment offsets within a stage, per K slice: fragment i
    // (rows 16 i on) adds the constant 16 i RB, as the swizzle depends only
    // on the row modulo 16.  The empty asm makes each offset one opaque
    // value, so every fragment address is the stage plus two terms; a deeper
    // chain of address arithmetic loses the per-array alias scope of the
    // stage, and the read then waits for every LDS load in flight.
    int offa[KSL], offb[KSL];
#pragma unroll
    for (int kk = 0; kk < KSL; ++kk) {
        offa[kk] = swz_k<KC>(wr * TM + lr, kk * 4 + lg);
        offb[kk] = BM * RB + swz_k<KC>(wc * TN + lr, kk * 4 + lg);
        asm("" : "+v"(offa[kk]));
        asm("" : "+v"(offb[kk]));
    }
    auto compute = [&](const unsigned char *A, unsigned char *next, bool refill) {
        uint4 af[KSL][FM], bf[KSL][FN];
        auto read_a = [&](int kk, int i) {
            af[kk][i] = *reinterpret_cast<const uint4 *>(A + offa[kk] + i * 16 * RB);
        };
        auto read_b = [&](int kk) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[kk][j] = *reinterpret_cast<const uint4 *>(A + offb[kk] + j * 16 * RB);
        };
        read_b(0);
        read_a(0, 0);
        if constexpr (FM > 1) read_a(0, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, FN + (FM > 1 ? 2 : 1), 0);
#pragma unroll
        for (int kk = 0; kk < KSL; ++kk) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int j = 0; j < FN; ++j) mma_16x16x32(bf[kk][j], af[kk][i], acc[i][j], T{});
                __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
                const int g2 = kk * FM + i + 2;       // the A fragment two groups ahead
                if (g2 < KSL * FM) {
                    const int k2 = g2 / FM, i2 = g2 % FM;
                    if (i2 == 0) {
                        read_b(k2);
                        read_a(k2, i2);
                        __builtin_amdgcn_sched_group_barrier(0x100, FN + 1, 0);
                    } else {
                        read_a(k2, i2);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
                if (kk == 0 && i == FM - 1) {
                    if constexpr (STAGES == 2) {
                        if (refill) issue(next, true);
                    } else {
                        issue(next, refill);
                    }
                }
            }
        }
    };
    // One step: wait for this wave's loads of the stage, barrier, multiply
    // the first half of the stage, refill the stage read one step ago (its
    // address work then overlaps the MFMAs in flight), multiply the rest.
    // Stages are named arrays, so after inlining each access targets one
    // known LDS object.
    auto wait_own = [&]() {
        constexpr int N = (STAGES - 2) * LPS;
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    };
#define MICONV_DMA_STEP(CUR, NEXT, S)             \
    {                                             \
        wait_own();                               \
        lds_barrier();                            \
        compute(CUR, NEXT, (S) + STAGES - 1 < nsteps); \
    }

    if constexpr (STAGES == 2) {
        // Two stages: each step waits for every load in flight, so steps
        // past the end are simply skipped.
        if (0 < nsteps) issue(st0, true);
        for (int s = 0; s < nsteps; s += 2) {
            MICONV_DMA_STEP(st0, st1, s)
            if (s + 1 < nsteps) MICONV_DMA_STEP(st1, st0, s + 1)
        }
    } else {
        // Three or four stages.  Every step issues a refill, a dead one past
        // the last step, and the step count is rounded up to whole rounds of
        // stages (the extra steps multiply zeros), so that no path through
        // the loop differs in the loads it has in flight: where such paths
        // join, the compiler loses track of which stage each pending load
        // writes and waits for all of them before the next LDS read.  Each
        // step waits for its own stage only, the later stages still loading.
        const int nsp = (nsteps + STAGES - 1) / STAGES * STAGES;
        issue(st0, 0 < nsteps);
        issue(st1, 1 < nsteps);
        if constexpr (STAGES > 3) issue(st2, 2 < nsteps);
        for (int s = 0; s < nsp; s += STAGES) {
            if constexpr (STAGES == 3) {
                MICONV_DMA_STEP(st0, st2, s)
                MICONV_DMA_STEP(st1, st0, s + 1)
                MICONV_DMA_STEP(st2, st1, s + 2)
            } else {
                MICONV_DMA_STEP(st0, st3, s)
                MICONV_DMA_STEP(st1, st0, s + 1)
                MICONV_DMA_STEP(st2, st1, s + 2)
                MICONV_DMA_STEP(st3, st2, s + 3)
            }
        }
        // The dead loads of the last round still write LDS.
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
    }
#undef MICONV_DMA_STEP

    // ---- epilogue: lane holds 4 consecutive channels of one output position ----
    if (a.ksplit > 1) {
        // Partial sums of this K range, fp32, bias and rounding left to the
        // reduction.
        const int prow = a.rows - a.row0;
        float *P = a.part + ((int64_t)(ks * a.G + g) * a.phases + phase) * prow * a.cog_pad;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = a.row0 + m_tile * BM + wr * TM + i * 16 + lr;
            if (m >= a.rows) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int co = n_tile * BN + wc * TN + j * 16 + lg * 4;
                *reinterpret_cast<f32x4 *>(P + (int64_t)(m - a.row0) * a.cog_pad + co) = acc[i][j];
            }
        }
        return;
    }
    T *__restrict__ Y = static_cast<T *>(a.y);
    const T *__restrict__ Bias = static_cast<const T *>(a.b);
    float bias[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int co = n_tile * BN + wc * TN + j * 16 + lg * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            bias[j][e] = (a.has_bias && co + e < a.Cog) ? to_f32(Bias[g * a.Cog + co + e]) : 0.f;
    }
    if constexpr (ES == 2) {
        if (a.y_lin) {
            // Rows of y are linear (row m at m * y_rs): the tile is staged in
            // LDS as [row][channel] and leaves as whole 16-byte chunks, lanes
            // on consecutive chunks of a row, so every store covers whole
            // lines; non-temporal, as nothing here reads y again and the L2
            // keeps the gathered input rows the next taps re-read.  Chunks of
            // a staged row are XOR-swizzled by the row so that the 16 rows
            // one staging write covers spread over the banks.  Rows go through
            // in passes of what the stages hold.
            constexpr int RBY = 2 * BN;                       // staged row bytes
            constexpr int CPR = BN / 8;                       // chunks per row (a power of two)
            constexpr int RPS = STAGE_BYTES / RBY;            // staged rows per stage array
            constexpr int PR0 = STAGES * RPS < BM ? STAGES * RPS : BM;
            constexpr int PR = PR0 / 16 * 16;                 // rows per pass
            static_assert(PR >= 16 && (CPR & (CPR - 1)) == 0, "staging geometry");
            auto srow = [&](int r) -> unsigned char * {
                const int si = r / RPS;
                // Only the stage arrays this instance has (si < STAGES).
                unsigned char *base = si == 0 ? st0
                                      : (si == 1 || STAGES == 2) ? st1
                                      : (si == 2 || STAGES == 3) ? st2
                                                                 : st3;
                return base + (r - si * RPS) * RBY;
            };
            const int mbase = a.row0 + m_tile * BM;
            T *ytile = Y + (int64_t)mbase * a.y_rs + g * a.Cog + n_tile * BN;
            __syncthreads();
            for (int p0 = 0; p0 < BM; p0 += PR) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wr * TM + i * 16 + lr - p0;
                    if (r < 0 || r >= PR) continue;
                    unsigned char *row = srow(r);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int c = (wc * TN + j * 16 + lg * 4) >> 3;
                        uint2 u;
                        u.x = pack2<T>(acc[i][j][0] + bias[j][0], acc[i][j][1] + bias[j][1]);
                        u.y = pack2<T>(acc[i][j][2] + bias[j][2], acc[i][j][3] + bias[j][3]);
                        *reinterpret_cast<uint2 *>(row + ((c ^ (r & (CPR - 1))) << 4) + ((lg & 1) << 3)) = u;
                    }
                }
                __syncthreads();
                for (int idx = tid; idx < PR * CPR; idx += 64 * NW) {
                    const int r = idx / CPR, c = idx & (CPR - 1);
                    if (p0 + r < BM && mbase + p0 + r < a.rows && n_tile * BN + 8 * c < a.Cog) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(srow(r) + ((c ^ (r & (CPR - 1))) << 4));
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<u32x4 *>(ytile + (int64_t)(p0 + r) * a.y_rs + 8 * c));
                    }
                }
                if (p0 + PR < BM) __syncthreads();
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = a.row0 + m_tile * BM + wr * TM + i * 16 + lr;
        if (m >= a.rows) continue;
        const int n = m / JJ;
        const int r = m - n * JJ;
        int q0 = r / J12;
        const int r2 = r - q0 * J12;
        int q1 = r2 / a.J[2], q2 = r2 - q1 * a.J[2];
        if (a.transposed) {
            q0 = a.S[0] * q0 + rho0;
            q1 = a.S[1] * q1 + rho1;
            q2 = a.S[2] * q2 + rho2;
            if (q0 >= a.O[0] || q1 >= a.O[1] || q2 >= a.O[2]) continue;
        }
        const int64_t yrow = (int64_t)n * a.ys_n + q0 * a.ys_l[0] + q1 * a.ys_l[1] + q2 * a.ys_l[2];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int co = n_tile * BN + wc * TN + j * 16 + lg * 4;
            const int cg = g * a.Cog + co;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e] + bias[j][e];
            T *dst = Y + yrow + (int64_t)cg * a.ys_c;
            if (a.y_vec4) {
                if (co < a.Cog) {
                    uint2 u;
                    u.x = pack2<T>(v[0], v[1]);
                    u.y = pack2<T>(v[2], v[3]);
                    *reinterpret_cast<uint2 *>(dst) = u;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (co + e < a.Cog) dst[(int64_t)e * a.ys_c] = from_f32<T>(v[e]);
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// Split-K reduction: y = bias + sum over the K ranges of the fp32 partial
// sums, rounded once; one thread per 4 consecutive output channels of one
// row (of one group and phase), stored at y's strides like the epilogue.
template <typename T>
__global__ __launch_bounds__(256) void igemm_splitk_reduce(IgArgs a)
{
    const int quads = (a.Cog + 3) / 4;
    const int prow = a.rows - a.row0;
    const int64_t total = (int64_t)a.G * a.phases * prow * quads;
    const int64_t plane = (int64_t)a.G * a.phases * prow * a.cog_pad;   // one K range
    T *__restrict__ Y = static_cast<T *>(a.y);
    const T *__restrict__ Bias = static_cast<const T *>(a.b);
    const int JJ = a.J[0] * a.J[1] * a.J[2];
    const int J12 = a.J[1] * a.J[2];
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int qd = (int)(idx % quads);
        int64_t r0 = idx / quads;
        const int mr = (int)(r0 % prow);
        r0 /= prow;
        const int phase = (int)(r0 % a.phases);
        const int g = (int)(r0 / a.phases);
        const int co = qd * 4;
        const float *P = a.part + (((int64_t)g * a.phases + phase) * prow + mr) * a.cog_pad + co;
        f32x4 s = *reinterpret_cast<const f32x4 *>(P);
        for (int k = 1; k < a.ksplit; ++k) s += *reinterpret_cast<const f32x4 *>(P + k * plane);
        const int m = a.row0 + mr;
        const int n = m / JJ;
        const int r = m - n * JJ;
        int q0 = r / J12;
        const int r2 = r - q0 * J12;
        int q1 = r2 / a.J[2], q2 = r2 - q1 * a.J[2];
        if (a.transposed) {
            int p = phase;
            const int rho2 = p % a.S[2];
            p /= a.S[2];
            const int rho1 = p % a.S[1];
            const int rho0 = p / a.S[1];
            q0 = a.S[0] * q0 + rho0;
            q1 = a.S[1] * q1 + rho1;
            q2 = a.S[2] * q2 + rho2;
            if (q0 >= a.O[0] || q1 >= a.O[1] || q2 >= a.O[2]) continue;
        }
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = s[e] + ((a.has_bias && co + e < a.Cog) ? to_f32(Bias[g * a.Cog + co + e]) : 0.f);
        T *dst = Y + (int64_t)n * a.ys_n + q0 * a.ys_l[0] + q1 * a.ys_l[1] + q2 * a.ys_l[2] +
                 (int64_t)(g * a.Cog + co) * a.ys_c;
        if (a.y_vec4) {
            uint2 u;
            u.x = pack2<T>(v[0], v[1]);
            u.y = pack2<T>(v[2], v[3]);
            *reinterpret_cast<uint2 *>(dst) = u;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (co + e < a.Cog) dst[(int64_t)e * a.ys_c] = from_f32<T>(v[e]);
        }
    }
}

// Weight repack: w (any strides) -> [G][Cog_pad][taps][Cig_pad], zero padded.
// One thread per 16-byte chunk of a packed row (Cig_pad is a multiple of the
// chunk): 32-bit index arithmetic (the packed weights stay below 2 GiB, the
// planner checks) once per chunk, the chunk's elements gathered at w's
// strides and stored as one vector.
template <typename T>
__global__ void igemm_repack(const T *__restrict__ w, T *__restrict__ wr, int32_t chunks, int32_t Cig, int32_t Cog,
                             int32_t cig_pad, int32_t cog_pad, int32_t taps, int32_t K1, int32_t K2, int64_t ws0,
                             int64_t ws1, int64_t wk0, int64_t wk1, int64_t wk2, int32_t transposed)
{
    constexpr int EV = 16 / sizeof(T);
    const int cpr = cig_pad / EV;   // chunks per packed row (g, j, t)
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += gridDim.x * blockDim.x) {
        const int cc = q % cpr;
        int r = q / cpr;
        const int t = r % taps;
        r /= taps;
        const int j = r % cog_pad;
        const int g = r / cog_pad;
        T v[EV];
        __builtin_memset(v, 0, sizeof(v));
        if (j < Cog) {
            const int t2 = t % K2, t1 = (t / K2) % K1, t0 = t / (K2 * K1);
            const int64_t toff = t0 * wk0 + t1 * wk1 + t2 * wk2;
            // Forward: w[g*Cog + j][c][t]; transposed: w[g*Cig + c][j][t].
            const int64_t base = transposed ? (int64_t)g * Cig * ws0 + (int64_t)j * ws1 + toff
                                            : ((int64_t)g * Cog + j) * ws0 + toff;
            const int64_t sc = transposed ? ws0 : ws1;
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int c = cc * EV + e;
                if (c < Cig) v[e] = w[base + (int64_t)c * sc];
            }
        }
        uint4 u;
        __builtin_memcpy(&u, v, 16);
        reinterpret_cast<uint4 *>(wr)[q] = u;
    }
}

namespace {

// eff: per-tile throughput relative to config 0 (measured throughput times the
// launch's rounds of workgroups over its exact rounds of work, dense 3x3 and
// transposed 1-D bf16 workloads on MI355X); the planner's cost estimate.
constexpr IgemmCfg kCfgs[] = {
    {256, 256, 64, 2, 4, 2, 100},  // 0: 8 waves, wave tile 128 x 64
    {160, 256, 64, 2, 2, 3, 72},   // 1: 4 waves, wave tile 80 x 128
    {128, 128, 64, 2, 2, 4, 53},   // 2: 4 waves, wave tile 64 x 64
    {256, 64, 64, 4, 1, 3, 50},    // 3: 4 waves, N <= 64
    {256, 32, 64, 4, 1, 3, 45},    // 4: 4 waves, N <= 32
    {128, 64, 32, 2, 2, 2, 100},   // 5: fp32 (register-staged path only)
    {128, 256, 64, 2, 2, 3, 70},   // 6: 4 waves, wave tile 64 x 128
    {256, 128, 64, 2, 2, 3, 60},   // 7: 4 waves, wave tile 128 x 64
    {128, 128, 64, 2, 2, 2, 100},  // 8: 4 waves, two stages: two workgroups per CU
    {256, 256, 32, 2, 4, 4, 93},   // 9: 8 waves, K step 32, 4 stages (deeper prefetch)
    {256, 256, 32, 2, 4, 3, 88},   // 10: 8 waves, K step 32, 3 stages
    {64, 256, 64, 1, 8, 3, 40},    // 11: 8 waves, wave tile 64 x 32 (rows left after the full rounds)
};

// Weight repack through an LDS tile, for weights whose packed rows (g, j, t)
// lie closer together in w than the channels c of one row -- the contiguous
// transposed weight [C_in][Cog][k] (rows adjacent, channels Cog*k apart), or
// the forward [C_out][Cig][k] with taps innermost.  A workgroup takes 64
// packed rows x 64 channels: lanes on consecutive rows read w (consecutive
// addresses where the rows are adjacent), the tile is transposed in LDS, and
// lanes on consecutive 16-byte chunks of each packed row write it.
template <typename T>
__global__ __launch_bounds__(256) void igemm_repack_t(const T *__restrict__ w, T *__restrict__ wr, int32_t nrows,
                                                     int32_t Cig, int32_t Cog, int32_t cig_pad, int32_t cog_pad,
                                                     int32_t taps, int32_t K1, int32_t K2, int64_t ws0, int64_t ws1,
                                                     int64_t wk0, int64_t wk1, int64_t wk2, int32_t transposed)
{
    constexpr int EV = 16 / sizeof(T);
    __shared__ T tile[64][65];
    const int tid = threadIdx.x;
    const int ctiles = cig_pad / 64;
    const int r0 = (blockIdx.x / ctiles) * 64, c0 = (blockIdx.x % ctiles) * 64;
    // Read: lane tr = packed row r0 + tr, channels c0 + tc, tc + 4, ...
    {
        const int tr = tid & 63, tc = tid >> 6;
        const int R = r0 + tr;
        int64_t base = 0;
        bool ok = R < nrows;
        if (ok) {
            const int t = R % taps;
            const int gj = R / taps;
            const int j = gj % cog_pad, g = gj / cog_pad;
            ok = j < Cog;
            const int t2 = t % K2, t1 = (t / K2) % K1, t0 = t / (K2 * K1);
            const int64_t toff = t0 * wk0 + t1 * wk1 + t2 * wk2;
            base = transposed ? (int64_t)g * Cig * ws0 + (int64_t)j * ws1 + toff : ((int64_t)g * Cog + j) * ws0 + toff;
        }
        const int64_t sc = transposed ? ws0 : ws1;
        // All sixteen reads in flight before the first LDS write.
        T v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int cc = c0 + tc + 4 * k;
            v[k] = (ok && cc < Cig) ? w[base + (int64_t)cc * sc] : T{};
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) tile[tc + 4 * k][tr] = v[k];
    }
    __syncthreads();
    // Write: 64 rows x 64 / EV chunks; lane -> (row, chunk), chunks fastest.
    constexpr int CPT = 64 / EV;
    for (int q = tid; q < 64 * CPT; q += 256) {
        const int r = q / CPT, ch = q % CPT;
        if (r0 + r >= nrows) continue;
        T v[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e) v[e] = tile[ch * EV + e][r];
        uint4 u;
        __builtin_memcpy(&u, v, 16);
        reinterpret_cast<uint4 *>(wr + (int64_t)(r0 + r) * cig_pad + c0)[ch] = u;
    }
}

template <typename T, int V, bool VEC>
hipError_t launch_cfg(const IgArgs &a, hipStream_t s)
{
    constexpr IgemmCfg c = kCfgs[V];
    if constexpr (VEC && Dt<T>::size == 2) {
        // Static LDS only (stages are separate arrays).
        hipLaunchKernelGGL((igemm_dma_kernel<T, c.bm, c.bn, c.wm, c.wn, c.stages, c.bk / 8>), dim3(a.total_tiles),
                           dim3(64 * c.wm * c.wn), 0, s, a);
    } else {
        const size_t lds = (size_t)2 * (c.bm + c.bn) * 128;
        auto kern = igemm_kernel<T, c.bm, c.bn, c.wm, c.wn, VEC>;
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(kern, dim3(a.total_tiles), dim3(64 * c.wm * c.wn), lds, s, a);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const IgArgs &a, int variant, bool vec, hipStream_t s)
{
    if constexpr (Dt<T>::size == 4) {
        return vec ? launch_cfg<T, 5, true>(a, s) : launch_cfg<T, 5, false>(a, s);
    } else {
        switch (variant) {
        case 0: return vec ? launch_cfg<T, 0, true>(a, s) : launch_cfg<T, 0, false>(a, s);
        case 1: return vec ? launch_cfg<T, 1, true>(a, s) : launch_cfg<T, 1, false>(a, s);
        case 2: return vec ? launch_cfg<T, 2, true>(a, s) : launch_cfg<T, 2, false>(a, s);
        case 3: return vec ? launch_cfg<T, 3, true>(a, s) : launch_cfg<T, 3, false>(a, s);
        case 4: return vec ? launch_cfg<T, 4, true>(a, s) : launch_cfg<T, 4, false>(a, s);
        case 6: return vec ? launch_cfg<T, 6, true>(a, s) : launch_cfg<T, 6, false>(a, s);
        case 7: return vec ? launch_cfg<T, 7, true>(a, s) : launch_cfg<T, 7, false>(a, s);
        case 8: return vec ? launch_cfg<T, 8, true>(a, s) : launch_cfg<T, 8, false>(a, s);
        case 9: return vec ? launch_cfg<T, 9, true>(a, s) : launch_cfg<T, 9, false>(a, s);
        case 10: return vec ? launch_cfg<T, 10, true>(a, s) : launch_cfg<T, 10, false>(a, s);
        case 11: return vec ? launch_cfg<T, 11, true>(a, s) : launch_cfg<T, 11, false>(a, s);
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
    const int64_t chunks = total / (16 / (int64_t)sizeof(T));
    // Packed rows (g, j, t) are taps-fastest; the stride of the innermost
    // tap, and the channel stride, in w.
    const int64_t row_stride = r > 0 ? wk[r - 1] : 1;
    const int64_t ch_stride = d.transposed ? d.w.strides[0] : d.w.strides[1];
    const int64_t nrows = total / p.tile[IG_CIG_PAD];
    if (row_stride < ch_stride && p.tile[IG_CIG_PAD] % 64 == 0 && nrows < (int64_t)1 << 30) {
        const int64_t blocks = cdiv(nrows, 64) * (p.tile[IG_CIG_PAD] / 64);
        hipLaunchKernelGGL((igemm_repack_t<T>), dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const T *>(w),
                           static_cast<T *>(ws), (int32_t)nrows, (int32_t)(d.C_in / d.groups),
                           (int32_t)(d.C_out / d.groups), (int32_t)p.tile[IG_CIG_PAD], (int32_t)p.tile[IG_COG_PAD],
                           (int32_t)taps, (int32_t)d.k[1], (int32_t)d.k[2], d.w.strides[0], d.w.strides[1], wk[0],
                           wk[1], wk[2], d.transposed);
        return hipGetLastError();
    }
    const int64_t blocks = std::min<int64_t>(cdiv(chunks, 256), 4096);
    hipLaunchKernelGGL((igemm_repack<T>), dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const T *>(w),
                       static_cast<T *>(ws), (int32_t)chunks, (int32_t)(d.C_in / d.groups), (int32_t)(d.C_out / d.groups),
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
    a.xs_n = (int32_t)d.x.strides[0];
    a.xs_c = (int32_t)d.x.strides[1];
    a.ys_n = p.y.strides[0];
    a.ys_c = p.y.strides[1];
    for (int i = 0; i < 3; ++i) {
        const bool on = i < r;
        a.xs_l[i] = on ? (int32_t)d.x.strides[2 + i] : 0;
        a.ys_l[i] = on ? p.y.strides[2 + i] : 0;
        a.L[i] = (int32_t)d.in[i];
        a.K[i] = (int32_t)d.k[i];
        a.O[i] = (int32_t)d.out[i];
        a.S[i] = (int32_t)d.stride[i];
        a.PB[i] = (int32_t)d.padding_before[i];
        a.D[i] = (int32_t)d.dilation[i];
        a.J[i] = (int32_t)(d.transposed ? cdiv(d.out[i], d.stride[i]) : d.out[i]);
    }
    a.x_bytes = (int32_t)p.tile[IG_XBYTES];
    a.Cig = (int32_t)(d.C_in / d.groups);
    a.Cog = (int32_t)(d.C_out / d.groups);
    a.cig_pad = (int32_t)p.tile[IG_CIG_PAD];
    a.cog_pad = (int32_t)p.tile[IG_COG_PAD];
    a.taps = (int32_t)(d.k[0] * d.k[1] * d.k[2]);
    a.G = (int32_t)d.groups;
    a.phases = (int32_t)p.tile[IG_PHASES];
    a.m_tiles = (int32_t)p.tile[IG_MTILES];
    a.n_tiles = (int32_t)p.tile[IG_NTILES];
    a.rows = (int32_t)p.tile[IG_ROWS];
    a.transposed = d.transposed;
    a.has_bias = d.has_bias;
    a.total_tiles = (int32_t)p.grid[0];
    a.w_bytes = (int32_t)igemm_wbytes(d.groups, p.tile[IG_COG_PAD], a.taps, p.tile[IG_CIG_PAD], esize(d.dtype));
    // Linear 16-byte output rows: a forward 16-bit call whose y is dense
    // channels-last (row m at m * C_out), channel counts in whole 8-channel
    // chunks, y 16-byte aligned.
    {
        bool lin = !d.transposed && esize(d.dtype) == 2 && p.y.strides[1] == 1 && d.C_out % 8 == 0 &&
                   (d.C_out / d.groups) % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
        int64_t e = d.C_out;
        for (int i = r - 1; i >= 0 && lin; --i) {
            lin = d.out[i] == 1 || p.y.strides[2 + i] == e;
            e *= d.out[i];
        }
        lin = lin && (d.N == 1 || p.y.strides[0] == e);
        a.y_lin = lin ? 1 : 0;
        a.y_rs = (int32_t)d.C_out;
    }
    // 4 consecutive output channels form one aligned vector in y.
    a.y_vec4 = (p.y.strides[1] == 1 && (reinterpret_cast<uintptr_t>(y) & (4 * esize(d.dtype) - 1)) == 0 &&
                p.y.strides[0] % 4 == 0 && (r < 1 || p.y.strides[2] % 4 == 0) &&
                (r < 2 || p.y.strides[3] % 4 == 0) && (r < 3 || p.y.strides[4] % 4 == 0) &&
                (d.C_out / d.groups) % 4 == 0)
                   ? 1
                   : 0;

    a.row0 = 0;

    a.one = (p.flags & CONV_PLAN_ONE_BY_ONE) && vec ? 1 : 0;
    hipError_t e = hipSuccess;
    if (p.flags & CONV_PLAN_ONE_BY_ONE) {
        // The weight tensor is the packed B operand: read in place.
        a.w = w;
        a.w_bytes = (int32_t)(d.C_out * d.C_in * esize(d.dtype));
    } else {
        switch (d.dtype) {
        case CONV_F32: e = launch_repack<float>(p, w, ws, s); break;
        case CONV_F16: e = launch_repack<f16_t>(p, w, ws, s); break;
        default: e = launch_repack<bf16_t>(p, w, ws, s); break;
        }
    }
    if (e != hipSuccess) return CONV_EDEVICE;
    if (p.variant == IG_T1_CFG || p.variant == IG_T1B_CFG) {
        // Both phases per workgroup; it needs the 16-byte loads of x (conv_run
        // sends a misaligned x to the phase-split tile), and writes y at any
        // element alignment.
        if (reinterpret_cast<uintptr_t>(x) & 15) return CONV_EALIGN;
        return launch_igemm_t1(p, x, ws, b, y, stream);
    }
    auto run = [&](const IgArgs &args, int variant) {
        switch (d.dtype) {
        case CONV_F32: return launch_typed<float>(args, variant, vec, s);
        case CONV_F16: return launch_typed<f16_t>(args, variant, vec, s);
        default: return launch_typed<bf16_t>(args, variant, vec, s);
        }
    };
    a.ksplit = 1;
    a.part = nullptr;
    const int64_t tail = p.tile[IG_TAIL];
    if (tail > 0) {
        // The planner split the rows: full-size tiles for whole rounds of
        // workgroups, then the rows left as 64-row tiles, their K split into
        // ksplit ranges whose fp32 partial sums a reduction adds up (with the
        // bias) -- so the rows that would leave most CUs idle in a last round
        // spread over all of them.
        const IgemmCfg &cm = igemm_cfg(p.variant);
        const int per_m = a.n_tiles * a.phases * a.G;
        IgArgs main = a;
        main.m_tiles = (int)(tail & 0xffffff);
        main.total_tiles = main.m_tiles * per_m;
        IgArgs t = a;
        t.row0 = main.m_tiles * cm.bm;
        t.m_tiles = (int)cdiv(a.rows - t.row0, igemm_cfg(IG_TAIL_CFG).bm);
        t.ksplit = vec ? (int)(tail >> 24) : 1;
        t.total_tiles = t.m_tiles * per_m * t.ksplit;
        if (t.ksplit > 1)
            t.part = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) +
                                               ((p.flags & CONV_PLAN_ONE_BY_ONE) ? 0 : a.w_bytes));
        e = main.m_tiles > 0 ? run(main, p.variant) : hipSuccess;
        if (e == hipSuccess) e = run(t, IG_TAIL_CFG);
        if (e == hipSuccess && t.ksplit > 1) {
            const int64_t total = (int64_t)a.G * a.phases * (a.rows - t.row0) * ((a.Cog + 3) / 4);
            const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 8192);
            switch (d.dtype) {
            case CONV_F16: hipLaunchKernelGGL((igemm_splitk_reduce<f16_t>), dim3(blocks), dim3(256), 0, s, t); break;
            default: hipLaunchKernelGGL((igemm_splitk_reduce<bf16_t>), dim3(blocks), dim3(256), 0, s, t); break;
            }
            e = hipGetLastError();
        }
    } else {
        e = run(a, p.variant);
    }
    return e == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
