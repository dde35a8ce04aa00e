// Transposed 1-D convolution with stride 2 on the matrix cores, both output
// phases in one workgroup (kernel CONV_K_IGEMM_T, plan variant IG_T1_CFG).
//
// executorch PR #25091 ("Run transposed convolutions on the implicit-GEMM
// template"), description, second paragraph: output o of a transposed
// convolution reads, at tap t, input (o + pb - t*dil)/s when that quotient is
// an exact integer inside the input.  With s = 2 and o = 2j + rho the
// quotient is  j + delta(rho, t),  delta = (rho + pb - t*dil)/2, exact only
// for the taps whose numerator is even; each tap belongs to exactly one
// phase rho.  Both phases of a block of rows j therefore read the same input
// rows, shifted by a few positions:
//
//   y[n, g*Cog + co, 2j + rho] = b + sum_{t of phase rho} sum_c
//                                    x[n, g*Cig + c, j + delta(rho, t)] * w[g*Cig + c, co, t]
//
// Tile: 256 rows j of one image x 64 output channels x both phases (512
// consecutive outputs o).  For each 32-channel block of K the workgroup loads
// ONE halo tile of x -- input rows j0 + delta_min .. j0 + delta_min + 319,
// out-of-range rows as zeros (the padding) -- and the block's weights for
// every tap, by direct-to-LDS buffer loads.  Each of the 4 waves owns one
// phase and 128 rows and multiplies, tap by tap, the halo rows shifted by
// that tap's delta against the tap's weights (v_mfma_f32_16x16x32, lane =
// 4 consecutive rows j of one output channel).  Input rows are read once per
// block, not once per (tap, phase), so x crosses HBM once.
//
// Two LDS stages of ~37 KB: two workgroups share a CU, so one's barrier and
// load waits overlap the other's matrix work.
//
// Epilogue: the 64 x 512 output tile (bias added in fp32, rounded once) is
// staged in LDS as [channel][o] and written along whichever of y's dims has
// stride 1.  For a contiguous [N, C, L] output each channel row is staged
// shifted by its own offset from a 16-byte boundary of y (rows of an odd
// length start at every even offset), so the row leaves as 16-byte chunks
// aligned to y -- one non-temporal store per lane -- plus the few elements
// of its two partial end chunks.
#include "dev_common.h"
#include "internal.h"

#include <algorithm>

namespace miconv {

struct T1Args {
    const void *x;
    const void *w;   // repacked weights [G][cog_pad][K][cig_pad]
    const void *b;
    void *y;
    int64_t ys_n, ys_c, ys_l;
    int32_t xs_n, xs_l;          // element strides of x (channel stride 1)
    int32_t x_bytes, w_bytes;
    int32_t L, O, N, G, Cig, Cog, cig_pad, cog_pad;
    int32_t pb, dil, dmin, span;   // smallest halo shift, and largest minus smallest
    int32_t jtiles, ntiles, total_tiles, has_bias, co_fast;
};

namespace {

// Geometry of one instance: NW waves (half per phase), each owning FM
// 16-row fragments of rows j and the tile's 64 output channels.
constexpr int T1_BN = 64;                   // output channels per tile
constexpr int T1_RB = 64;                   // LDS row bytes: 32 channels of 16-bit
constexpr int t1_fm(int nw) { return nw == 4 ? 8 : 7; }
constexpr int t1_bm(int nw) { return nw / 2 * 16 * t1_fm(nw); }             // rows j per tile
constexpr int t1_hr(int nw) { return (t1_bm(nw) + 64 + 16 * nw - 1) / (16 * nw) * (16 * nw); }  // halo rows
// Staging row bytes: the row, up to 7 elements of shift, and an odd number of
// dwords in all, so that the 16 channel rows one staging write covers fall on
// distinct banks.
constexpr int t1_sr(int nw) { return 2 * (2 * t1_bm(nw)) + 20; }
constexpr int t1_ab(int nt, int nw) { return t1_hr(nw) * T1_RB + nt * T1_BN * T1_RB; }
// A stage holds the halo and the weights, and at the end whole staging rows:
// all stages together hold the 64 channel rows of the output tile.
constexpr int t1_stage_bytes(int nt, int nw, int stages)
{
    const int need_rows = (T1_BN + stages - 1) / stages;
    const int ab = t1_ab(nt, nw);
    return ab > need_rows * t1_sr(nw) ? ab : need_rows * t1_sr(nw);
}

}  // namespace

int igemm_t1_lds_bytes(int taps, int variant)
{
    return variant == IG_T1_CFG ? 2 * t1_stage_bytes(taps, 4, 2) : 3 * t1_stage_bytes(taps, 8, 3);
}
int igemm_t1_rows(int variant) { return variant == IG_T1_CFG ? t1_bm(4) : t1_bm(8); }

// Two workgroups per CU where their LDS fits (four waves, up to 80 KB).
constexpr int t1_wgs_per_cu(int nt, int nw, int stages)
{
    return nw == 4 && stages * t1_stage_bytes(nt, nw, stages) <= 80 * 1024 ? 2 : 1;
}

// REG: an even number of taps and an odd dilation, so each phase owns
// exactly NT/2 taps, every other one (t = t0, t0 + 2, ...): the fragment
// reads of a step then form one static stream over the wave's taps.
template <typename T, int NT, int NW, int STAGES, bool REG>
__global__ __launch_bounds__(NW * 64, t1_wgs_per_cu(NT, NW, STAGES)) void igemm_t1_kernel(T1Args a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int ES = 2;
    constexpr int BN = T1_BN, RB = T1_RB;
    constexpr int FM = t1_fm(NW), FN = 4;     // wave tile 16*FM rows x 64 channels
    constexpr int WR = 16 * FM;               // rows j per wave
    constexpr int BM = t1_bm(NW), HR = t1_hr(NW), SR = t1_sr(NW);
    constexpr int A_BYTES = HR * RB;
    constexpr int STAGE_BYTES = t1_stage_bytes(NT, NW, STAGES);
    constexpr int RPS = STAGE_BYTES / SR;     // staging rows per stage
    constexpr int A_IT = HR / (16 * NW);      // A loads per wave per step (16 rows each)
    constexpr int B_IT = NT * BN / (16 * NW); // B loads per wave per step
    constexpr int LPS = A_IT + B_IT;
    static_assert(HR % (16 * NW) == 0 && (NT * BN) % (16 * NW) == 0, "loads per wave");
    static_assert(RPS * STAGES >= BN, "staging rows");
    static_assert(STAGES == 2 || STAGES == 3, "stages");

    __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st2[STAGES > 2 ? STAGE_BYTES : 16];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int tile = xcd_tile(blockIdx.x, a.total_tiles);
    // Tile order (fastest first): channel tile, row tile, image, group -- the
    // channel tiles that read the same halo rows run side by side on one XCD.
    const int n_tile = tile % a.ntiles;
    int rest = tile / a.ntiles;
    const int jt = rest % a.jtiles;
    rest /= a.jtiles;
    const int n = rest % a.N;
    const int g = rest / a.N;
    const int j0 = jt * BM;

    // ---- direct-to-LDS load offsets: instruction q of wave w fills LDS rows
    // (NW*q + w)*16 + lane/4, slot lane%4, with the logical 8-channel chunk the
    // swizzle puts in that slot ----
    const int lrow = lane >> 2;
    int a_off[A_IT], a_kc[A_IT];
#pragma unroll
    for (int q = 0; q < A_IT; ++q) {
        const int row = (NW * q + wave) * 16 + lrow;
        const int kc = (lane & 3) ^ ((row >> 1) & 3);
        const int i = j0 + a.dmin + row;           // input position of halo row `row`
        a_kc[q] = kc;
        // Rows past the tile's last shifted row are never read: not loaded.
        const bool used = row < BM + a.span;
        a_off[q] = used && (unsigned)i < (unsigned)a.L ? (n * a.xs_n + i * a.xs_l + g * a.Cig + kc * 8) * ES
                                                       : 0x7fffff00;
    }
    int b_off[B_IT];
#pragma unroll
    for (int q = 0; q < B_IT; ++q) {
        const int row = (NW * q + wave) * 16 + lrow;   // tap * 64 + column
        const int kc = (lane & 3) ^ ((row >> 1) & 3);
        const int t = row / BN, col = row % BN;
        b_off[q] = (((g * a.cog_pad + n_tile * BN + col) * NT + t) * a.cig_pad + kc * 8) * ES;
    }
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.x), (short)0, a.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.w), (short)0, a.w_bytes, 0x00020000);
    typedef __attribute__((address_space(3))) void *lds_ptr;
    const bool cig_full = a.Cig % 32 == 0;

    // Loads of channel block cb into stage S (the block rides in the scalar
    // offset; chunks past Cig read zeros).  A dead issue (past the last
    // block) loads out of range everywhere: it fills the stage with zeros
    // and keeps every step's count of loads in flight the same.
    auto issue = [&](unsigned char *S, int cb, bool live) {
        const int soff = cb * 32 * ES;
#pragma unroll
        for (int q = 0; q < A_IT; ++q) {
            const bool cok = live && (cig_full || cb * 32 + a_kc[q] * 8 < a.Cig);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(S + (NW * q + wave) * 16 * RB), 16,
                                                     cok ? a_off[q] : 0x7fffff00, soff, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < B_IT; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(S + A_BYTES + (NW * q + wave) * 16 * RB), 16,
                                                     live ? b_off[q] : 0x7fffff00, soff, 0, 0);
    };

    const int rho = wave & 1, wr = wave >> 1;
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This lane's fragment offsets.  A fragment i of a tap with halo shift h
    // is rows wr*WR + 16i + h + (0..15); the swizzle repeats every 16 rows,
    // so fragment i adds the constant 16*i*RB to the offset of fragment 0.
    // B fragment jj of tap t is rows t*64 + 16*jj + (0..15).  Each offset is
    // made opaque so that every fragment address is the stage plus one
    // per-lane value and a constant (the stage array keeps its alias scope and
    // the reads wait only for the loads of that stage).
    int offb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        offb[t] = A_BYTES + swz_k<4>(t * BN + lr, lg);
        asm("" : "+v"(offb[t]));
    }
    // The regular case: this wave's taps t_u = t0 + 2u and their halo
    // shifts are known before the K loop, so each tap's A and B fragment
    // offsets are computed once.  The reads run as one stream interleaved with
    // the MFMAs (as in the forward tile): the first tap's B fragments and
    // first two A fragments up front, then after each group of FN MFMAs the
    // A fragment two groups ahead -- with, where that fragment opens the next
    // tap, that tap's B fragments -- pinned by scheduling groups.
    constexpr int TPH = REG ? NT / 2 : 1;
    int offa_r[TPH], offb_r[TPH];
    if constexpr (REG) {
        const int t0 = (rho + a.pb) & 1;
#pragma unroll
        for (int u = 0; u < TPH; ++u) {
            const int t = t0 + 2 * u;
            const int h = ((rho + a.pb - t * a.dil) >> 1) - a.dmin;
            offa_r[u] = swz_k<4>(wr * WR + lr + h, lg);
            offb_r[u] = A_BYTES + swz_k<4>(t * BN + lr, lg);
            asm("" : "+v"(offa_r[u]));
            asm("" : "+v"(offb_r[u]));
        }
    }
    auto compute_reg = [&](const unsigned char *S) {
        uint4 af[TPH][FM], bf[TPH][FN];
        auto read_a = [&](int u, int i) { af[u][i] = *reinterpret_cast<const uint4 *>(S + offa_r[u] + i * 16 * RB); };
        auto read_b = [&](int u) {
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) bf[u][jj] = *reinterpret_cast<const uint4 *>(S + offb_r[u] + jj * 16 * RB);
        };
        read_b(0);
        read_a(0, 0);
        read_a(0, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, FN + 2, 0);
#pragma unroll
        for (int u = 0; u < TPH; ++u) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) mma_16x16x32(af[u][i], bf[u][jj], acc[i][jj], T{});
                __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
                const int g2 = u * FM + i + 2;
                if (g2 < TPH * FM) {
                    const int u2 = g2 / FM, i2 = g2 % FM;
                    if (i2 == 0) {
                        read_b(u2);
                        read_a(u2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, FN + 1, 0);
                    } else {
                        read_a(u2, i2);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
            }
        }
    };
    auto compute = [&](const unsigned char *S) {
        if constexpr (REG) {
            compute_reg(S);
            return;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int num = rho + a.pb - t * a.dil;
            if (num & 1) continue;                      // tap of the other phase (wave-uniform)
            const int h = (num >> 1) - a.dmin;
            int offa = swz_k<4>(wr * WR + lr + h, lg);
            asm("" : "+v"(offa));
            uint4 af[FM], bf[FN];
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) bf[jj] = *reinterpret_cast<const uint4 *>(S + offb[t] + jj * 16 * RB);
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const uint4 *>(S + offa + i * 16 * RB);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) mma_16x16x32(af[i], bf[jj], acc[i][jj], T{});
        }
    };
    auto wait_all = [&]() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); };   // vmcnt(0)

    const int nsteps = a.cig_pad / 32;
    if constexpr (STAGES == 2) {
        // ---- K loop over 32-channel blocks, two stages: the loads of block
        // s+1 are issued right after the barrier that opens block s (every
        // wave has then finished reading the stage they overwrite) ----
        if (nsteps > 0) issue(st0, 0, true);
        for (int s = 0; s < nsteps; s += 2) {
            wait_all();
            lds_barrier();
            if (s + 1 < nsteps) issue(st1, s + 1, true);
            compute(st0);
            if (s + 1 < nsteps) {
                wait_all();
                lds_barrier();
                if (s + 2 < nsteps) issue(st0, s + 2, true);
                compute(st1);
            }
        }
    } else {
        // ---- three stages: block s+2 is loaded while block s is multiplied;
        // each step waits only for its own stage's loads (the next stage's
        // stay in flight).  Every step issues its refill, a dead one past the
        // last block, so every path has the same loads in flight ----
        auto wait_own = [&]() {
            __builtin_amdgcn_s_waitcnt((LPS & 15) | (7 << 4) | (15 << 8) | ((LPS >> 4) << 14));
        };
        issue(st0, 0, 0 < nsteps);
        issue(st1, 1, 1 < nsteps);
#define MICONV_T1_STEP(CUR, NEXT, S)            \
    {                                           \
        wait_own();                             \
        lds_barrier();                          \
        issue(NEXT, (S) + 2, (S) + 2 < nsteps); \
        if ((S) < nsteps) compute(CUR);         \
    }
        for (int s = 0; s < nsteps; s += 3) {
            MICONV_T1_STEP(st0, st2, s)
            MICONV_T1_STEP(st1, st0, s + 1)
            MICONV_T1_STEP(st2, st1, s + 2)
        }
#undef MICONV_T1_STEP
    }

    // ---- epilogue: stage [channel][o] in LDS (RPS channel rows per stage),
    // then write along y's unit-stride dim ----
    //
    // Positions contiguous in y (pvec): each channel row of the tile is
    // staged shifted by sh, the offset in elements of its first output from
    // a 16-byte boundary of y, so that LDS chunk q of the row is exactly the
    // 16-byte-aligned chunk q of y's row segment; full chunks then leave as
    // single 16-byte stores and only the two partial end chunks element by
    // element.  (Rows of an odd length start at every even byte offset.)
    wait_all();
    __syncthreads();
    T *__restrict__ Y = static_cast<T *>(a.y);
    const int o0 = 2 * j0;
    const int cbase = g * a.Cog + n_tile * BN;
    const int64_t ybase = (int64_t)n * a.ys_n + (int64_t)cbase * a.ys_c + (int64_t)o0 * a.ys_l;
    const bool pvec = !a.co_fast && a.ys_l == 1;
    auto shift_of = [&](int col) -> int {
        const uint64_t addr = reinterpret_cast<uintptr_t>(Y) + 2 * (uint64_t)(ybase + (int64_t)col * a.ys_c);
        return pvec ? (int)((addr & 15) >> 1) : 0;
    };
    auto srow = [&](int col) -> unsigned char * {
        const int sidx = col / RPS, r = col - sidx * RPS;
        unsigned char *base = sidx == 0 ? st0 : (sidx == 1 ? st1 : st2);
        return base + r * SR;
    };
    const T *__restrict__ Bias = static_cast<const T *>(a.b);
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
        const int col = 16 * jj + lr;
        const float bias = (a.has_bias && n_tile * BN + col < a.Cog) ? to_f32(Bias[cbase + col]) : 0.f;
        unsigned char *row = srow(col) + 2 * shift_of(col);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ol = 2 * (wr * WR + 16 * i + 4 * lg + e) + rho;
                *reinterpret_cast<T *>(row + 2 * ol) = from_f32<T>(acc[i][jj][e] + bias);
            }
    }
    __syncthreads();
    const int ncol = min(BN, a.Cog - n_tile * BN), nout = min(2 * BM, a.O - o0);
    if (pvec) {
        // Full chunks first: wave w takes channel rows w, w+NW, ..., four at a
        // time (their staged reads in flight together), lane l chunks l,
        // l+64, ...; chunk q is full when outputs 8q - sh .. 8q - sh + 7 all
        // lie in [0, nout).  The stores are non-temporal: whole lines that
        // nothing here reads again, kept out of the L2 that holds the
        // weights and the halo rows the neighbouring channel tiles share.
        constexpr int NQ = 2 * BM / 8;           // chunks per row that can be full
        for (int c0 = wave; c0 < ncol; c0 += 4 * NW) {
            u32x4 v[4][(NQ + 63) / 64];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = c0 + r * NW;
                const unsigned char *row = srow(col < ncol ? col : 0);
#pragma unroll
                for (int h = 0; h < (NQ + 63) / 64; ++h)
                    if (64 * h + lane < NQ) {
                        // Rows start on 4-byte boundaries: four dword reads.
                        const uint32_t *src = reinterpret_cast<const uint32_t *>(row + 16 * (64 * h + lane));
                        v[r][h] = u32x4{src[0], src[1], src[2], src[3]};
                    }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = c0 + r * NW;
                if (col >= ncol) break;
                const int sh = shift_of(col);
                unsigned char *ab = reinterpret_cast<unsigned char *>(Y + ybase + (int64_t)col * a.ys_c) - 2 * sh;
#pragma unroll
                for (int h = 0; h < (NQ + 63) / 64; ++h) {
                    const int q = 64 * h + lane, first = 8 * q - sh;
                    if (q < NQ && first >= 0 && first + 8 <= nout)
                        __builtin_nontemporal_store(v[r][h], reinterpret_cast<u32x4 *>(ab + 16 * q));
                }
            }
        }
        // Then the partial chunks at each row's two ends, element by element:
        // the head, outputs [0, hd) before the first chunk boundary, and the
        // tail, outputs [8 ql - sh, nout) after the last full chunk.  Thread
        // t takes slots t, t + 64 NW, ...: slot = 16 row + k, k < 8 the head's
        // k-th output, k >= 8 the tail's (k-8)-th.
        for (int slot = tid; slot < ncol * 16; slot += 64 * NW) {
            const int col = slot >> 4, k = slot & 15;
            const int sh = shift_of(col);
            const int hd = min((8 - sh) & 7, nout), ql = (nout + sh) >> 3;
            const int o = k < 8 ? k : max(8 * ql - sh, hd) + (k - 8);
            if ((k < 8 && o < hd) || (k >= 8 && o < nout)) {
                const T e = *reinterpret_cast<const T *>(srow(col) + 2 * (o + sh));
                Y[ybase + (int64_t)col * a.ys_c + o] = e;
            }
        }
    } else if (!a.co_fast) {
        // Positions fastest at a stride: wave w writes channel rows w, w+NW,
        // ..., lane l elements l, l+64, ... of a row, eight staged reads in
        // flight before their eight stores.
        for (int col = wave; col < ncol; col += NW) {
            const unsigned char *row = srow(col);
            T *dst = Y + ybase + (int64_t)col * a.ys_c;
            for (int c0 = 0; c0 < 2 * BM; c0 += 8 * 64) {
                T v[8];
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    if (c0 + 64 * c < 2 * BM) v[c] = *reinterpret_cast<const T *>(row + 2 * (c0 + 64 * c + lane));
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int ol = c0 + 64 * c + lane;
                    if (c0 + 64 * c < 2 * BM && ol < nout) dst[(int64_t)ol * a.ys_l] = v[c];
                }
            }
        }
    } else {
        // Channels fastest: lane l is channel l, wave w writes positions
        // w*(2*BM/NW) onwards.
        const unsigned char *row = srow(lane);
        T *dst = Y + ybase + (int64_t)lane * a.ys_c;
        constexpr int PW = 2 * BM / NW;
        for (int p0 = wave * PW; p0 < wave * PW + PW; p0 += 8) {
            T v[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = *reinterpret_cast<const T *>(row + 2 * (p0 + c));
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (lane < ncol && p0 + c < nout) dst[(int64_t)(p0 + c) * a.ys_l] = v[c];
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// Halo-tile geometry of a call: the smallest shift delta over all taps, and
// whether the shifts span at most 64 rows.
namespace {

template <typename T, int NT, int NW, int STAGES>
void t1_launch(const T1Args &a, bool reg, dim3 grid, hipStream_t s)
{
    if constexpr (NT % 2 == 0) {
        if (reg) {
            hipLaunchKernelGGL((igemm_t1_kernel<T, NT, NW, STAGES, true>), grid, dim3(NW * 64), 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((igemm_t1_kernel<T, NT, NW, STAGES, false>), grid, dim3(NW * 64), 0, s, a);
}

}  // namespace

bool igemm_t1_shifts(const conv_desc &d, int *dmin, int *span)
{
    int lo = 1 << 30, hi = -(1 << 30);
    for (int rho = 0; rho < 2; ++rho)
        for (int64_t t = 0; t < d.k[0]; ++t) {
            const int64_t num = rho + d.padding_before[0] - t * d.dilation[0];
            if (num & 1) continue;
            const int64_t delta = num >> 1;
            lo = (int)std::min<int64_t>(lo, delta);
            hi = (int)std::max<int64_t>(hi, delta);
        }
    if (lo > hi) lo = hi = 0;
    *dmin = lo;
    if (span) *span = hi - lo;
    return hi - lo <= 64;
}

int launch_igemm_t1(const conv_plan_t &p, const void *x, const void *wpacked, const void *b, void *y, void *stream)
{
    const conv_desc &d = p.d;
    T1Args a;
    a.x = x;
    a.w = wpacked;
    a.b = b;
    a.y = y;
    a.ys_n = p.y.strides[0];
    a.ys_c = p.y.strides[1];
    a.ys_l = p.y.strides[2];
    a.xs_n = (int32_t)d.x.strides[0];
    a.xs_l = (int32_t)d.x.strides[2];
    a.x_bytes = (int32_t)p.tile[IG_XBYTES];
    a.L = (int32_t)d.in[0];
    a.O = (int32_t)d.out[0];
    a.N = (int32_t)d.N;
    a.G = (int32_t)d.groups;
    a.Cig = (int32_t)(d.C_in / d.groups);
    a.Cog = (int32_t)(d.C_out / d.groups);
    a.cig_pad = (int32_t)p.tile[IG_CIG_PAD];
    a.cog_pad = (int32_t)p.tile[IG_COG_PAD];
    a.pb = (int32_t)d.padding_before[0];
    a.dil = (int32_t)d.dilation[0];
    int dmin = 0, span = 0;
    igemm_t1_shifts(d, &dmin, &span);
    a.dmin = dmin;
    a.span = span;
    const bool big = p.variant != IG_T1_CFG;
    a.jtiles = (int32_t)cdiv(cdiv(d.out[0], 2), big ? t1_bm(8) : t1_bm(4));
    a.ntiles = (int32_t)p.tile[IG_NTILES];
    a.total_tiles = (int32_t)p.grid[0];
    a.has_bias = d.has_bias;
    a.co_fast = (p.y.strides[1] == 1 && p.y.strides[2] != 1) ? 1 : 0;
    a.w_bytes = (int32_t)igemm_wbytes(d.groups, p.tile[IG_COG_PAD], d.k[0], p.tile[IG_CIG_PAD], 2);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)p.grid[0]);
    const int k = (int)d.k[0];
    // Eight waves and three stages for 2 or 4 taps (the weights of a step
    // split evenly over eight waves, three stages within the LDS); four waves
    // and two stages otherwise.
    // Even tap counts with an odd dilation take the static read stream.
    const bool reg = k % 2 == 0 && (d.dilation[0] & 1);
#define MICONV_T1(K_)                                                                 \
    case K_:                                                                          \
        if (big) {                                                                    \
            if constexpr (K_ == 2 || K_ == 4) {                                       \
                if (d.dtype == CONV_F16)                                              \
                    t1_launch<f16_t, K_, 8, 3>(a, reg, grid, s);                      \
                else                                                                  \
                    t1_launch<bf16_t, K_, 8, 3>(a, reg, grid, s);                     \
            } else {                                                                  \
                return CONV_EUNSUPPORTED;                                             \
            }                                                                         \
        } else if (d.dtype == CONV_F16) {                                             \
            t1_launch<f16_t, K_, 4, 2>(a, reg, grid, s);                              \
        } else {                                                                      \
            t1_launch<bf16_t, K_, 4, 2>(a, reg, grid, s);                             \
        }                                                                             \
        break;
    switch (k) {
        MICONV_T1(2) MICONV_T1(3) MICONV_T1(4) MICONV_T1(5) MICONV_T1(6) MICONV_T1(7) MICONV_T1(8)
    default: return CONV_EUNSUPPORTED;
    }
#undef MICONV_T1
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_EDEVICE;
}

}  // namespace miconv
