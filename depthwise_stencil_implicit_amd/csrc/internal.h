// Host-side internals shared by the binding, planner and launcher.
#pragma once

#include <cstdint>

#include "../../include/miconv.h"

namespace miconv {

// Output length of one spatial dim (< 1 means no valid output).
int64_t out_len(int transposed, int64_t L, int64_t k, int64_t s, int64_t pb, int64_t pa, int64_t dil,
                int64_t op);

// Channels-last-like and not also contiguous-like.
bool channels_last_like(const conv_tensor &t);

// Batched output descriptor of a canonical call.
void batched_out(const conv_desc &d, conv_tensor &y);

inline int64_t esize(int32_t dtype) { return dtype == CONV_F32 ? 4 : 2; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Grouped-stencil schedules (kernel CONV_K_GRP, plan.variant): the vector
// dot2 schedules, or the matrix-core plane schedule for small 3x3 groups
// whose planes are contiguous.
enum { GRP_SCHED_VALU = 0, GRP_SCHED_MMA = 1 };

// Implicit GEMM schedule table (kernel CONV_K_IGEMM / CONV_K_IGEMM_T).
struct IgemmCfg {
    int bm, bn, bk;     // workgroup tile: rows, columns, K per step
    int wm, wn;         // waves along rows / columns (block = 64 * wm * wn)
    int stages;         // LDS stages of the direct-to-LDS pipeline
    int eff;            // measured relative MFMA throughput of the schedule, percent
};
const IgemmCfg &igemm_cfg(int variant);
int igemm_num_cfgs();
// The 64-row schedule that runs the rows a sparse last round would leave to a
// few CUs; the planner does not choose it for whole calls.
constexpr int IG_TAIL_CFG = 11;
// Transposed 1-D calls with stride 2: both output phases per workgroup from
// one halo tile of input rows (a kernel of its own, not a table entry).
constexpr int IG_T1_CFG = 12;   // four waves, two stages, 256 rows j per tile
constexpr int IG_T1B_CFG = 13;  // eight waves, three stages, 448 rows j (2 or 4 taps)
// Smallest halo shift of such a call and the spread of the shifts (span may
// be NULL); false when they spread over more than the kernel's 64 spare halo
// rows.
bool igemm_t1_shifts(const conv_desc &d, int *dmin, int *span);
int igemm_t1_lds_bytes(int taps, int variant);
int igemm_t1_rows(int variant);

// Plan-field indices for the implicit GEMM (plan.tile[]).
// IG_TAIL: 0, or (row tiles of the full-size launch) | (K ranges of the
// 64-row launch that covers the remaining rows) << 24.
enum { IG_CIG_PAD = 0, IG_COG_PAD = 1, IG_PHASES = 2, IG_MTILES = 3, IG_NTILES = 4, IG_ROWS = 5, IG_XBYTES = 6,
       IG_TAIL = 7 };
// CUs the planner assumes when it sizes the implicit GEMM's rounds of
// workgroups (MI355X; the plan makes no device calls).
constexpr int kIgCus = 256;
// Bytes of the repacked weights at the start of the workspace.
inline int64_t igemm_wbytes(int64_t groups, int64_t cog_pad, int64_t taps, int64_t cig_pad, int64_t es)
{
    return (groups * cog_pad * taps * cig_pad * es + 255) / 256 * 256;
}

// Depthwise channels-last stencil (kernel CONV_K_DW_CL).  A workgroup of 256
// threads owns CW consecutive 32-bit channel words, OCOLS consecutive output
// columns and one block of output rows of one image; thread t is channel word
// t % CW of the strip of DW_TO output columns t / CW.  Input rows are shared
// by the workgroup through a ring of D rows in LDS, filled by direct-to-LDS
// loads of CB bytes per lane (LPW instructions per wave per row).  Finished
// output rows are staged in LDS (two buffers) and written with CB-byte stores,
// DW_NS per wave per row, in the step after the one that finished them.
// Before reading a ring row a wave waits until at most the VMEM instructions
// issued after that row's loads are pending: the loads of the D-2 rows after
// it and the stores of the D-1 steps before it.
constexpr int DW_TO = 7;
constexpr int dw_cw(int S) { return S == 1 ? 32 : 64; }
constexpr int dw_ocols(int S) { return 256 / dw_cw(S) * DW_TO; }
constexpr int dw_icols(int K, int S) { return (dw_ocols(S) - 1) * S + K; }
constexpr int dw_lpw(int K, int S, int CB) { return (dw_icols(K, S) * (dw_cw(S) * 4 / CB) + 255) / 256; }
constexpr int dw_ns(int S, int CB) { return (dw_ocols(S) * (dw_cw(S) * 4 / CB) + 255) / 256; }
constexpr int dw_row_bytes(int K, int S, int CB) { return dw_lpw(K, S, CB) * 256 * CB; }
constexpr int dw_stage_bytes(int S) { return dw_ocols(S) * dw_cw(S) * 4; }
// LDS after the ring: the two staging buffers, which first hold the
// workgroup's weights (CW words x K*K taps of 4 bytes per word).
constexpr int dw_tail_bytes(int K, int S)
{
    return 2 * dw_stage_bytes(S) > dw_cw(S) * 4 * K * K ? 2 * dw_stage_bytes(S) : dw_cw(S) * 4 * K * K;
}
constexpr int dw_pending(int K, int S, int CB, int D)
{
    return (D - 2) * dw_lpw(K, S, CB) + ((D - 1 + S - 1) / S) * dw_ns(S, CB);
}
// Workgroups resident per CU: three for the light stride-1 stencils (k3, and
// k5 on the 16-byte path, fit 12 waves per CU in registers, and a 4-row ring
// keeps three rings in LDS), one for k9 at stride 1 (its nine open output rows
// of accumulators take more than half the registers), two with a 6-row ring
// otherwise.
constexpr int dw_wgs_per_cu(int K, int S, int CB)
{
    return S == 1 && (K == 3 || (K == 5 && CB == 16)) ? 3 : (K == 9 && S == 1 ? 1 : 2);
}
constexpr int dw_depth(int K, int S, int CB)
{
    int d = dw_wgs_per_cu(K, S, CB) == 3 ? 4 : 6;
    while (d > 3 && (dw_pending(K, S, CB, d) > 63 || d * dw_row_bytes(K, S, CB) + dw_tail_bytes(K, S) > 80 * 1024))
        --d;
    return d;
}
constexpr int dw_lds_bytes(int K, int S, int CB)
{
    return dw_depth(K, S, CB) * dw_row_bytes(K, S, CB) + dw_tail_bytes(K, S);
}
// Plan-field indices for the depthwise stencil (plan.tile[]).
// dw_cl plan variants: 0 = ring kernel with 4-byte accesses, 1 = ring kernel
// with 16-byte accesses, DWCL_GENERIC = the generic schedule (any multiplier,
// kernel shape and stride; no LDS).
constexpr int DWCL_GENERIC = 2;
enum { DW_CW = 0, DW_OCOLS = 1, DW_CHCHUNKS = 2, DW_COLCHUNKS = 3, DW_XBYTES = 4, DW_YBYTES = 5, DW_RBLOCKS = 6,
       DW_RPB = 7 };

// Weight-gradient schedule fields (conv_bwd_plan_t.wg_tile[]): WB_MFMA is 0
// for the simple kernel, WB_DW for the depthwise stencil (channel words of
// channels-last operands), else 1 | 2 (P read position-major) | 4 (Q read
// position-major) for the matrix-core one; padded a / b extents, ranges of
// positions (of rows of positions for WB_DW), and the byte ranges of the two
// operands for the 16-byte loads.
enum { WB_MFMA = 0, WB_APAD = 1, WB_BPAD = 2, WB_SPLITS = 3, WB_PBYTES = 4, WB_QBYTES = 5, WB_GYCL = 6 };
// WB_GYCL (conv_bwd_plan_t.wg_tile[6]): bytes of a channels-last copy of a
// channel-major gy at the start of the workspace (0: gy is read as given).
// The gradients of a call with channels-last x then read gy channels-last
// too: the 16-byte implicit-GEMM and matrix-core weight-gradient paths.
inline void channels_last_of(const conv_tensor &t, conv_tensor &o)
{
    o = t;
    int64_t acc = t.sizes[1];
    o.strides[1] = 1;
    for (int i = t.rank - 1; i >= 2; --i) {
        o.strides[i] = acc;
        acc *= t.sizes[i];
    }
    o.strides[0] = acc;
}
constexpr int64_t WB_DW = 8;
// Tap groups of the depthwise weight-gradient stencil: a workgroup holds
// 256 / TG channel words x TG groups of taps, fewer groups for small kernels
// so that one gy word feeds more taps.
inline int wgrad_dw_tg(int64_t taps) { return taps <= 16 ? 2 : (taps <= 28 ? 4 : 8); }
// WB_PLANE: forward calls on channel-major operands (each (image, channel)
// plane of x and gy dense), few channels per group: a workgroup per (group,
// range of images) stages each image's planes in LDS as fp32 and a thread per
// (output channel, input channel, tap) walks the positions.
constexpr int64_t WB_PLANE = 16;
// LDS of that schedule: the group's gy planes plus its x planes with the
// padding as a zero halo, fp32.
inline int64_t wgrad_plane_lds(const conv_desc &d)
{
    const int64_t Cig = d.C_in / d.groups, Cog = d.C_out / d.groups;
    int64_t pos = 1, halo = 1;
    for (int i = 0; i < d.spatial; ++i) {
        pos *= d.out[i];
        halo *= d.in[i] + d.padding_before[i] + d.padding_after[i];
    }
    return (Cog * pos + Cig * halo) * 4;
}

// The bias gradient by rows: gy's channel stride is not 1 and every image's
// channel plane is one dense run of at least 64 positions (channel-major gy),
// so a workgroup per (image, channel) reads its run with consecutive lanes;
// the ranges of the partial sums are then the images.
inline bool bgrad_by_rows(const conv_desc &d, const conv_tensor &gy)
{
    if (gy.strides[1] == 1) return false;
    int64_t acc = 1;
    for (int i = d.spatial - 1; i >= 0; --i) {
        if (d.out[i] > 1 && gy.strides[2 + i] != acc) return false;
        acc *= d.out[i];
    }
    return acc >= 64 && d.N <= 65536;
}

// The channels-last copy of a channel-major gy (each (image, channel) plane
// one dense run of L positions), into dst.
int launch_gy_to_cl(const conv_bwd_plan_t &p, const void *gy, void *dst, void *stream);

// Launchers (defined in the .hip files).  `vec` selects the 16-byte path.
int launch_igemm(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *ws,
                 void *stream, bool vec);
int launch_igemm_t1(const conv_plan_t &p, const void *x, const void *wpacked, const void *b, void *y,
                    void *stream);
int launch_plane(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream);
// The plan of n images of a plan that runs its batch in chunks
// (conv_plan_t.batch_chunk).
int plan_batch_part(const conv_plan_t &whole, int64_t n, conv_plan_t *out);
int launch_dwcl(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream,
                bool vec);
int launch_grp(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream);
int launch_wgrad(const conv_bwd_plan_t &p, const void *x, const void *gy, void *dw, void *ws, void *stream);
int launch_bgrad(const conv_bwd_plan_t &p, const void *gy, void *db, void *ws, void *stream);
int launch_fill_zero(void *out, const conv_tensor &t, void *stream);
// The weight reversed along every tap dim with its two channel dims exchanged
// per group, contiguous [C_in][C_out/groups][k...], into dst (the stride-1
// input gradient's forward call).
int launch_flip_weight(const conv_bwd_plan_t &p, const void *w, void *dst, void *stream);
int launch_reduce(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream);

}  // namespace miconv
