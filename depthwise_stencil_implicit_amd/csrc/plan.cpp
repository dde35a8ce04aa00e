// conv_plan: route a canonical call to a kernel and fix its launch.
//
// executorch PR #25084 ("Add triton::convolution and the conv routing
// framework"), description: each template declares what it supports, tests
// can force one schedule, and the planner refuses calls whose output layout
// differs from the one the op computes.
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: depthwise and
// up-to-8-input-channel grouped 2-D convolutions with dilation 1 and kernels up
// to 9x9 go to the direct stencil; grouped calls with a wide per-group product
// stay on the GEMM path.
// executorch PR #25091 ("Run transposed convolutions on the implicit-GEMM
// template"), description: transposed calls run on the implicit GEMM with the
// transposed gather.
//
// Routing (host only, deterministic):
//   transposed depthwise (multiplier 1, dil 1, k <= 9, r <= 2, column
//     stride <= 2), channel-contiguous x              -> DW_CL (generic)
//   other transposed                                  -> IGEMM_T
//   r <= 2, dil 1, k <= 9, groups > 1, Cig <= 8:
//       few outputs (<= 4 positions, >= 32 taps each) -> REDUCE
//       depthwise, channel-contiguous x and y          -> DW_CL
//         (ring kernels for multiplier 1 and a compiled square (k, s);
//          the generic schedule for any multiplier, shape and stride)
//       grouped (Cig even), fp16/bf16                  -> GRP
//       otherwise                                      -> PLANE
//   everything else                                   -> IGEMM
#include <cstring>
#include <algorithm>
#include <initializer_list>

#include "internal.h"

namespace miconv {
bool dwcl_has_schedule(int64_t kh, int64_t kw, int64_t sh, int64_t sw);
bool grp_supported(const conv_desc &d);
bool grp_geometry(const conv_desc &d, conv_plan_t &p);
bool grp_fits(const conv_desc &d);
void reduce_geometry(const conv_desc &d, conv_plan_t &p);
}  // namespace miconv

namespace {

using namespace miconv;

constexpr int64_t kLdsBudget = 64 * 1024;
constexpr int64_t kI32 = 0x7fffffffLL;

int64_t numel(const conv_tensor &t)
{
    int64_t n = 1;
    for (int i = 0; i < t.rank; ++i) n *= t.sizes[i];
    return n;
}

int64_t cig(const conv_desc &d) { return d.C_in / d.groups; }
int64_t cog(const conv_desc &d) { return d.C_out / d.groups; }

bool all_dil1(const conv_desc &d)
{
    for (int i = 0; i < d.spatial; ++i)
        if (d.dilation[i] != 1) return false;
    return true;
}

bool k_le(const conv_desc &d, int64_t kmax)
{
    for (int i = 0; i < d.spatial; ++i)
        if (d.k[i] > kmax) return false;
    return true;
}

bool sizes_fit_i32(const conv_desc &d)
{
    for (int i = 0; i < 3; ++i)
        if (d.in[i] > kI32 / 4 || d.out[i] > kI32 / 4 || d.k[i] > 4096 || d.stride[i] > 65536 ||
            d.dilation[i] > 65536 || d.padding_before[i] > kI32 / 4 || d.padding_after[i] > kI32 / 4)
            return false;
    return d.C_in < kI32 && d.C_out < kI32;
}

// ---------------------------------------------------------------- supports --

bool stencil_domain(const conv_desc &d)
{
    return !d.transposed && (d.spatial == 1 || d.spatial == 2) && cig(d) >= 1 && cig(d) <= 8 && k_le(d, 9);
}

// Byte span of a tensor (largest element offset + 1) times the element size.
int64_t span_bytes(const conv_tensor &t, int64_t es)
{
    int64_t off = 0;
    for (int i = 0; i < t.rank; ++i)
        if (t.sizes[i] > 0) off += (t.sizes[i] - 1) * t.strides[i];
    return (off + 1) * es;
}

// The generic channels-last depthwise schedule: any channel multiplier,
// kernel shape (within the stencil domain), any row stride and column
// strides 1..3, 1-D or 2-D, x and y
// channel-contiguous; 16-bit outputs leave as words of two channels, so y's
// position strides must keep channel pairs on 4-byte boundaries.
bool dwcl_generic_ok(const conv_desc &d, const conv_tensor &y)
{
    if (!stencil_domain(d) || !all_dil1(d)) return false;
    if (cig(d) != 1 || d.groups != d.C_in || d.C_out % d.C_in) return false;
    if (d.stride[d.spatial - 1] > 3) return false;   // compiled column strides 1..3
    if (d.x.strides[1] != 1) return false;
    // Buffer loads: non-negative strides, one image of x and the weight each
    // below 2^31 bytes.
    int64_t xi = 0, wi = 0;
    for (int i = 0; i < d.x.rank; ++i) {
        if (d.x.strides[i] < 0) return false;
        if (i > 0) xi += (d.x.sizes[i] - 1) * d.x.strides[i];
    }
    for (int i = 0; i < d.w.rank; ++i) {
        if (d.w.strides[i] < 0) return false;
        wi += (d.w.sizes[i] - 1) * d.w.strides[i];
    }
    if ((xi + 1) * esize(d.dtype) > kI32 - 4096 || (wi + 1) * esize(d.dtype) > kI32 - 4096) return false;
    // y channels-last (channel words), or with its positions contiguous (the
    // channel-major output ATen gives a 1-D call on a channels-last input).
    if (y.strides[1] == 1) {
        if (esize(d.dtype) == 2)
            for (int i = 0; i < y.rank; ++i)
                if (i != 1 && y.sizes[i] > 1 && y.strides[i] % 2) return false;
        return true;
    }
    return y.strides[y.rank - 1] == 1;
}

// The transposed generic schedule: transposed depthwise calls with
// multiplier 1, dilation 1, kernels up to 9 wide, column stride 1 or 2 (any
// row stride), 1-D or 2-D, channel-contiguous x, y at any non-negative
// strides (element stores).
bool dwcl_tgeneric_ok(const conv_desc &d, const conv_tensor &y)
{
    if (!d.transposed || (d.spatial != 1 && d.spatial != 2) || !all_dil1(d) || !k_le(d, 9)) return false;
    if (d.groups != d.C_in || d.C_out != d.C_in) return false;
    if (d.stride[d.spatial - 1] > 2) return false;
    if (d.x.strides[1] != 1) return false;
    for (const conv_tensor *t : {&d.x, &d.w, &y})
        for (int i = 0; i < t->rank; ++i)
            if (t->strides[i] < 0) return false;
    return true;
}

// The ring kernels: multiplier 1, a compiled square (k, s) schedule.
bool dwcl_ring_ok(const conv_desc &d, const conv_tensor &y)
{
    if (!stencil_domain(d) || d.spatial != 2 || !all_dil1(d)) return false;
    if (cig(d) != 1 || d.groups != d.C_in || d.C_out != d.C_in) return false;
    if (!dwcl_has_schedule(d.k[0], d.k[1], d.stride[0], d.stride[1])) return false;
    if (d.x.strides[1] != 1 || y.strides[1] != 1) return false;
    // One lane word holds 4 bytes of channels: word-aligned channel runs.
    const int64_t v = 4 / esize(d.dtype);
    if (d.C_in % v) return false;
    for (int i : {0, 2, 3})
        if (d.x.strides[i] % v || y.strides[i] % v) return false;
    // 32-bit buffer offsets for loads and stores.
    return span_bytes(d.x, esize(d.dtype)) <= kI32 - 4096 && span_bytes(y, esize(d.dtype)) <= kI32 - 4096;
}

bool supports_dwcl(const conv_desc &d, const conv_tensor &y)
{
    return dwcl_ring_ok(d, y) || dwcl_generic_ok(d, y) || dwcl_tgeneric_ok(d, y);
}

bool supports_plane(const conv_desc &d) { return stencil_domain(d); }

bool supports_reduce(const conv_desc &d) { return stencil_domain(d); }

bool supports_igemm(const conv_desc &d) { return !d.transposed; }
bool supports_igemm_t(const conv_desc &d) { return d.transposed != 0; }

bool few_outputs(const conv_desc &d)
{
    const int64_t positions = d.out[0] * d.out[1] * d.out[2];
    const int64_t taps = cig(d) * d.k[0] * d.k[1] * d.k[2];
    return positions <= 4 && taps >= 32;
}

int route(const conv_desc &d, const conv_tensor &y)
{
    if (d.transposed) return dwcl_tgeneric_ok(d, y) ? CONV_K_DW_CL : CONV_K_IGEMM_T;
    if (stencil_domain(d) && all_dil1(d) && d.groups > 1) {
        if (few_outputs(d)) return CONV_K_REDUCE;
        if (supports_dwcl(d, y)) return CONV_K_DW_CL;
        if (cig(d) >= 2 && grp_supported(d)) {
            // Every grouped schedule keeps the group's weights in LDS; a
            // wide per-group product that does not fit is a GEMM.
            if (!grp_fits(d)) return CONV_K_IGEMM;
            return CONV_K_GRP;
        }
        return CONV_K_PLANE;
    }
    return CONV_K_IGEMM;
}

// ---------------------------------------------------------------- geometry --

void geom_dwcl(const conv_desc &d, conv_plan_t &p, bool generic)
{
    if (generic) {
        // Lane = one word of output channels x DWG 8 output columns; a
        // workgroup = 32 words x 8 column strips of one output row.
        const int64_t v = esize(d.dtype) == 2 ? 2 : 1;
        const int64_t OH = d.spatial == 2 ? d.out[0] : 1, OW = d.out[d.spatial - 1];
        p.tile[DW_CHCHUNKS] = cdiv(cdiv(d.C_out, v), 32);
        p.tile[DW_COLCHUNKS] = cdiv(OW, 64);
        p.grid[0] = d.N * OH * p.tile[DW_COLCHUNKS] * p.tile[DW_CHCHUNKS];
        p.block = 256;
        p.variant = DWCL_GENERIC;
        p.lds_bytes = 0;
        p.vec_ok = 1;
        return;
    }
    const int k = (int)d.k[1], s = (int)d.stride[1];
    const int64_t es = esize(d.dtype);
    const int64_t words = d.C_in * es / 4;
    const int64_t cw = dw_cw(s);
    p.tile[DW_CW] = cw;
    p.tile[DW_OCOLS] = dw_ocols(s);
    p.tile[DW_CHCHUNKS] = cdiv(words, cw);
    p.tile[DW_COLCHUNKS] = cdiv(d.out[1], dw_ocols(s));
    p.tile[DW_XBYTES] = span_bytes(d.x, es);
    p.tile[DW_YBYTES] = span_bytes(p.y, es);
    // variant 1: 16-byte direct-to-LDS loads and 16-byte stores, which need
    // 16-byte aligned channel runs (x and y must also be 16-byte aligned at run
    // time; y is dense with x's channel count); variant 0 moves 4-byte channel
    // words.
    bool q = (d.C_in * es) % 16 == 0;
    for (int i : {0, 2, 3}) q = q && (d.x.strides[i] * es) % 16 == 0;
    // Row blocks: enough workgroups to fill every CU once (two or three per
    // CU), each one block of output rows of one image (no block crosses an
    // image).
    const int64_t tasks = d.N * p.tile[DW_CHCHUNKS] * p.tile[DW_COLCHUNKS];
    const int64_t want = 256 * dw_wgs_per_cu(k, s, q ? 16 : 4);
    int64_t rb = std::max<int64_t>(1, std::min<int64_t>(d.out[0], cdiv(want, std::max<int64_t>(tasks, 1))));
    const int64_t rpb = cdiv(d.out[0], rb);
    rb = cdiv(d.out[0], rpb);
    p.tile[DW_RBLOCKS] = rb;
    p.tile[DW_RPB] = rpb;
    p.grid[0] = tasks * rb;
    p.block = 256;
    p.variant = q ? 1 : 0;
    p.lds_bytes = dw_lds_bytes(k, s, q ? 16 : 4);
    p.vec_ok = 1;
}

bool geom_plane(const conv_desc &d, conv_plan_t &p)
{
    const bool two = d.spatial == 2;
    const int64_t OH = two ? d.out[0] : 1, OW = two ? d.out[1] : d.out[0];
    const int64_t KH = two ? d.k[0] : 1, KW = two ? d.k[1] : d.k[0];
    const int64_t SH = two ? d.stride[0] : 1, SW = two ? d.stride[1] : d.stride[0];
    const int64_t DH = two ? d.dilation[0] : 1, DW = two ? d.dilation[1] : d.dilation[0];
    int64_t TW, R, TH;
    if (!two) {
        TW = 256;
        R = 1;
        TH = 1;
    } else {
        TW = OW >= 48 ? 64 : (OW >= 24 ? 32 : 16);
        R = 2;
        TH = (256 / TW) * R;
    }
    auto lds = [&](int64_t th, int64_t tw) {
        const int64_t ih = (th - 1) * SH + (KH - 1) * DH + 1;
        const int64_t iw = (tw - 1) * SW + (KW - 1) * DW + 1;
        return cig(d) * ih * iw * 4;
    };
    while (lds(TH, TW) > kLdsBudget) {
        if (TH > R)
            TH /= 2;
        else if (TW > 1)
            TW /= 2;
        else
            return false;
    }
    if (TH % R) R = 1;
    const int64_t IH = (TH - 1) * SH + (KH - 1) * DH + 1;
    const int64_t IW = (TW - 1) * SW + (KW - 1) * DW + 1;
    int64_t mb = 1;
    while (mb < cog(d) && mb < 16) mb *= 2;
    p.tile[0] = TH;
    p.tile[1] = TW;
    p.tile[2] = R;
    p.tile[3] = mb;
    p.tile[4] = IH;
    p.tile[5] = IW;
    p.tile[6] = cdiv(OH, TH);
    p.tile[7] = cdiv(OW, TW);
    p.grid[0] = d.N * d.groups * p.tile[6] * p.tile[7];
    p.block = 256;
    p.lds_bytes = (int32_t)lds(TH, TW);
    return p.grid[0] <= kI32;
}

// Implicit GEMM: choose the tile shape with the least estimated CU time,
// rounds of workgroups over the 256 CUs times the tile area each runs.
bool geom_igemm(const conv_desc &d, conv_plan_t &p, int force_variant)
{
    int64_t phases = 1, rows = d.N;
    for (int i = 0; i < 3; ++i) {
        if (d.transposed) {
            phases *= d.stride[i];
            rows *= cdiv(d.out[i], d.stride[i]);
        } else {
            rows *= d.out[i];
        }
    }
    const int64_t es = esize(d.dtype);
    const int64_t xspan = span_bytes(d.x, es);
    // Element offsets into x are 32-bit in the kernel.
    if (xspan / es >= kI32 || rows >= kI32) return false;
    const int64_t cig_v = cig(d);
    // Transposed 1-D calls with stride 2 and channel-contiguous 16-byte chunks
    // of x: both output phases per workgroup from one halo tile of input rows.
    {
        int dmin = 0;
        const int64_t ev = 16 / es;
        const bool t1 = d.transposed && d.spatial == 1 && d.stride[0] == 2 && d.dtype != CONV_F32 && d.k[0] >= 2 &&
                        d.k[0] <= 8 && igemm_t1_shifts(d, &dmin, nullptr) && d.x.strides[1] == 1 && cig_v % ev == 0 &&
                        d.x.strides[0] % ev == 0 && d.x.strides[2] % ev == 0 && xspan < kI32 - 4096;
        const bool t1b = t1 && (d.k[0] == 2 || d.k[0] == 4);
        if ((force_variant == IG_T1_CFG && !t1) || (force_variant == IG_T1B_CFG && !t1b)) return false;
        if (t1 && (force_variant < 0 || force_variant == IG_T1_CFG || force_variant == IG_T1B_CFG)) {
            const int v = force_variant >= 0 ? force_variant : IG_T1_CFG;
            const int64_t cig_pad = round_up(cig_v, 64), cog_pad = round_up(cog(d) > 0 ? cog(d) : 1, 64);
            const int64_t J = cdiv(d.out[0], 2), jtiles = cdiv(J, igemm_t1_rows(v));
            p.variant = v;
            p.tile[IG_CIG_PAD] = cig_pad;
            p.tile[IG_COG_PAD] = cog_pad;
            p.tile[IG_PHASES] = 2;
            p.tile[IG_MTILES] = d.N * jtiles;
            p.tile[IG_NTILES] = cog_pad / 64;
            p.tile[IG_ROWS] = d.N * J;
            p.tile[IG_XBYTES] = xspan;
            p.tile[IG_TAIL] = 0;
            p.grid[0] = d.groups * d.N * jtiles * (cog_pad / 64);
            p.block = v == IG_T1_CFG ? 256 : 512;
            p.lds_bytes = igemm_t1_lds_bytes((int)d.k[0], v);
            p.workspace_bytes = igemm_wbytes(d.groups, cog_pad, d.k[0], cig_pad, es);
            p.vec_ok = 1;
            return p.workspace_bytes < kI32;
        }
    }
    int best = -1;
    double best_cost = 0;
    const int lo = d.dtype == CONV_F32 ? 5 : 0, hi = d.dtype == CONV_F32 ? 5 : igemm_num_cfgs() - 1;
    for (int v = lo; v <= hi; ++v) {
        if ((v == 5) != (d.dtype == CONV_F32) || v == IG_TAIL_CFG) continue;
        const IgemmCfg &c = igemm_cfg(v);
        const int64_t lds = (int64_t)c.stages * (c.bm + c.bn) * 128;
        const int64_t occ = lds > 80 * 1024 ? 1 : 2;
        const int64_t tiles = d.groups * phases * cdiv(rows, c.bm) * cdiv(cog(d) > 0 ? cog(d) : 1, c.bn);
        double rounds = (double)cdiv(tiles, kIgCus * occ);
        // A sparse last round of one-per-CU tiles runs split over all CUs (the
        // 64-row split-K launch below), at about a third of the efficiency.
        const IgemmCfg &ct = igemm_cfg(IG_TAIL_CFG);
        const int64_t left = tiles % kIgCus;
        if (occ == 1 && d.dtype != CONV_F32 && c.bm > ct.bm && c.bn == ct.bn && tiles > kIgCus && left > 0 &&
            4 * left <= kIgCus)
            rounds = (double)(tiles / kIgCus) + 3.0 * (double)left / kIgCus;
        // CU time of one resident round, over the schedule's measured efficiency.
        const double cost = rounds * occ * c.bm * c.bn / (double)c.eff;
        if (best < 0 || cost < best_cost) {
            best = v;
            best_cost = cost;
        }
    }
    // An explicit schedule (conv_plan_ex): a tile configuration of the same
    // dtype class, or the call is refused.
    if (force_variant >= 0) {
        if (force_variant < lo || force_variant >= igemm_num_cfgs() || (force_variant == 5) != (d.dtype == CONV_F32))
            return false;
        best = force_variant;
    }
    const IgemmCfg &c = igemm_cfg(best);
    const int64_t taps = d.k[0] * d.k[1] * d.k[2];
    // Channel padding: a multiple of every K step either kernel path may use
    // (the register-staged fallback steps 64 channels of 16-bit types, 32 of fp32).
    const int64_t cig_pad = round_up(cig(d), d.dtype == CONV_F32 ? 32 : 64);
    const int64_t cog_pad = round_up(cog(d) > 0 ? cog(d) : 1, c.bn);
    p.variant = best;
    p.tile[IG_CIG_PAD] = cig_pad;
    p.tile[IG_COG_PAD] = cog_pad;
    p.tile[IG_PHASES] = phases;
    p.tile[IG_MTILES] = cdiv(rows, c.bm);
    p.tile[IG_NTILES] = cog_pad / c.bn;
    p.tile[IG_ROWS] = rows;
    p.tile[IG_XBYTES] = xspan < kI32 - 4096 ? xspan : 0;
    p.grid[0] = d.groups * phases * p.tile[IG_MTILES] * p.tile[IG_NTILES];
    p.block = 64 * c.wm * c.wn;
    p.lds_bytes = (int32_t)(c.stages * (c.bm + c.bn) * 128);
    // A forward 1x1 call with stride 1 and no padding on dense channels-last
    // x (row m of the GEMM is x's pixel m) and a contiguous [C_out, C_in]
    // weight with C_in a multiple of the 64-channel block (then the weight
    // already has the packed layout): a plain GEMM, no repack, no position
    // arithmetic (Inductor conv.py, conv1x1_via_mm).
    bool one = !d.transposed && d.groups == 1 && d.dtype != CONV_F32 && cig(d) == cig_pad && taps == 1 &&
               d.x.strides[1] == 1 && d.w.strides[1] == 1 && d.w.strides[0] == d.C_in &&
               d.C_out * d.C_in * es < kI32 - 4096;
    {
        int64_t acc = d.C_in;
        for (int i = d.spatial - 1; i >= 0 && one; --i) {
            one = d.stride[i] == 1 && d.padding_before[i] == 0 && d.padding_after[i] == 0 &&
                  (d.in[i] == 1 || d.x.strides[2 + i] == acc);
            acc *= d.in[i];
        }
        one = one && (d.N == 1 || d.x.strides[0] == acc);
    }
    p.flags = one ? CONV_PLAN_ONE_BY_ONE : 0;
    p.workspace_bytes = one ? 0 : igemm_wbytes(d.groups, cog_pad, taps, cig_pad, es);
    if (p.workspace_bytes >= kI32) return false;   // 32-bit buffer offsets into the weights
    // Rows whose tiles would leave a last round that keeps at most a quarter
    // of the CUs busy go to 64-row tiles with their K split over the CUs
    // (fp32 partial sums in the workspace after the weights).
    p.tile[IG_TAIL] = 0;
    const IgemmCfg &ct = igemm_cfg(IG_TAIL_CFG);
    const int64_t per_m = p.tile[IG_NTILES] * phases * d.groups;
    const int64_t total = p.grid[0];
    const int64_t left = total % kIgCus;
    if (d.dtype != CONV_F32 && c.bm > ct.bm && c.bn == ct.bn && total > kIgCus && left > 0 && 4 * left <= kIgCus) {
        const int64_t m_tail = cdiv(left, per_m);
        const int64_t main_m = p.tile[IG_MTILES] - m_tail;
        const int64_t tail_rows = rows - main_m * c.bm;
        const int64_t tail_tiles = cdiv(tail_rows, ct.bm) * per_m;
        // Fewest K steps of any phase (valid taps x 64-channel blocks).
        int64_t min_taps = 1;
        for (int i = 0; i < d.spatial; ++i) {
            int64_t lo = d.k[i];
            if (d.transposed) {
                for (int64_t rho = 0; rho < d.stride[i]; ++rho) {
                    int64_t cnt = 0;
                    for (int64_t t = 0; t < d.k[i]; ++t)
                        if ((((rho + d.padding_before[i] - t * d.dilation[i]) % d.stride[i]) + d.stride[i]) % d.stride[i] == 0) ++cnt;
                    lo = std::min(lo, cnt);
                }
            }
            min_taps *= lo;
        }
        const int64_t min_steps = min_taps * (cig_pad / ct.bk);
        int64_t ks = std::max<int64_t>(1, std::min<int64_t>({8, kIgCus / std::max<int64_t>(tail_tiles, 1), min_steps}));
        p.tile[IG_TAIL] = main_m | (ks << 24);
        if (ks > 1) p.workspace_bytes += round_up(ks * d.groups * phases * tail_rows * cog_pad * 4, 256);
    }
    // 16-byte buffer-load path: contiguous, chunk-aligned channels, span < 2 GB.
    const int64_t ev = 16 / es;
    bool vec = d.x.strides[1] == 1 && cig(d) % ev == 0 && d.x.strides[0] % ev == 0 && p.tile[IG_XBYTES] > 0;
    for (int i = 0; i < d.spatial; ++i) vec = vec && d.x.strides[2 + i] % ev == 0;
    p.vec_ok = vec ? 1 : 0;
    return true;
}

// Algorithmic FLOPs: 2 per (output element, input channel, tap) term whose
// input index is an integer -- every tap for forward calls (padding-border
// taps included, the usual GEMM count), and for transposed calls only the taps
// whose numerator is divisible by the stride.
int64_t algorithmic_flops(const conv_desc &d)
{
    double terms = (double)d.N * (double)d.C_out * (double)cig(d);
    for (int i = 0; i < d.spatial; ++i) {
        if (!d.transposed) {
            terms *= (double)d.out[i] * (double)d.k[i];
        } else {
            int64_t cnt = 0;
            for (int64_t o = 0; o < d.out[i]; ++o)
                for (int64_t t = 0; t < d.k[i]; ++t)
                    if ((o + d.padding_before[i] - t * d.dilation[i]) % d.stride[i] == 0) ++cnt;
            terms *= (double)cnt;
        }
    }
    return (int64_t)(2.0 * terms);
}

bool same_layout(const conv_tensor &a, const conv_tensor &b)
{
    if (a.rank != b.rank || a.dtype != b.dtype) return false;
    for (int i = 0; i < a.rank; ++i) {
        if (a.sizes[i] != b.sizes[i]) return false;
        if (a.sizes[i] > 1 && a.strides[i] != b.strides[i]) return false;
    }
    return true;
}

}  // namespace

extern "C" int conv_plan_ex(const conv_desc *d, const conv_tensor *y, const conv_plan_opts *o, conv_plan_t *p)
{
    if (!d || !y || !p) return CONV_EINVAL;
    const int32_t force_kernel = o ? o->force_kernel : CONV_K_AUTO;
    const int32_t force_variant = o ? o->force_variant : -1;
    if (force_variant >= 0 && force_kernel != CONV_K_IGEMM && force_kernel != CONV_K_IGEMM_T &&
        force_kernel != CONV_K_GRP && force_kernel != CONV_K_DW_CL)
        return CONV_EINVAL;
    if (d->spatial < 1 || d->spatial > 3 || d->groups < 1 || d->x.rank != d->spatial + 2) return CONV_EINVAL;
    conv_tensor expect;
    if (conv_out_shape(d, &expect) != CONV_OK) return CONV_EINVAL;
    if (!same_layout(*y, expect)) return CONV_ELAYOUT;
    if (!sizes_fit_i32(*d)) return CONV_EUNSUPPORTED;

    // A batch whose x or y spans 2 GiB or more runs in chunks of images (the
    // kernels take 32-bit buffer offsets): the plan is a chunk's, with d and
    // y left the whole call, and conv_run steps through the batch.  The
    // workspace covers the last, smaller chunk as well.
    {
        conv_tensor yfull;
        batched_out(*d, yfull);
        const int64_t es = esize(d->dtype), lim = kI32 - 4096;
        if ((span_bytes(d->x, es) > lim || span_bytes(yfull, es) > lim) && d->N > 1 && !d->unbatched) {
            auto most = [&](const conv_tensor &t) -> int64_t {
                conv_tensor one = t;
                one.sizes[0] = 1;
                const int64_t img = span_bytes(one, es), st = t.strides[0] * es;
                if (st <= 0 || img > lim) return 0;
                return (lim - img) / st + 1;
            };
            const int64_t nc = std::min<int64_t>(std::min(most(d->x), most(yfull)), d->N);
            if (nc >= 1 && nc < d->N) {
                conv_desc cd = *d;
                conv_tensor cy = yfull;
                cd.N = nc;
                cd.x.sizes[0] = nc;
                cy.sizes[0] = nc;
                conv_plan_t cp;
                int st = conv_plan_ex(&cd, &cy, o, &cp);
                if (st != CONV_OK) return st;
                int64_t ws = cp.workspace_bytes;
                if (d->N % nc) {
                    conv_plan_t whole = cp;
                    whole.d = *d;
                    whole.y = yfull;
                    whole.batch_chunk = (int32_t)nc;
                    conv_plan_t rp;
                    st = plan_batch_part(whole, d->N % nc, &rp);
                    if (st != CONV_OK) return st;
                    ws = std::max(ws, rp.workspace_bytes);
                }
                cp.d = *d;
                cp.y = yfull;
                cp.batch_chunk = (int32_t)nc;
                cp.workspace_bytes = ws;
                cp.index64 = 1;
                cp.flops = algorithmic_flops(*d);
                cp.bytes = (numel(d->x) + numel(d->w) + (d->has_bias ? d->C_out : 0) + numel(yfull)) * es;
                *p = cp;
                return CONV_OK;
            }
        }
    }

    conv_plan_t plan;
    std::memset(&plan, 0, sizeof(plan));
    plan.d = *d;
    batched_out(*d, plan.y);
    const conv_tensor &yb = plan.y;

    int k = force_kernel;
    if (k == CONV_K_AUTO) {
        k = route(*d, yb);
    } else {
        bool ok;
        switch (k) {
        case CONV_K_DW_CL: ok = supports_dwcl(*d, yb); break;
        case CONV_K_PLANE: ok = supports_plane(*d); break;
        case CONV_K_GRP: ok = stencil_domain(*d) && grp_supported(*d) && grp_fits(*d); break;
        case CONV_K_REDUCE: ok = supports_reduce(*d); break;
        case CONV_K_IGEMM: ok = supports_igemm(*d); break;
        case CONV_K_IGEMM_T: ok = supports_igemm_t(*d); break;
        default: ok = false;
        }
        if (!ok) return CONV_EUNSUPPORTED;
    }
    plan.kernel = k;
    switch (k) {
    case CONV_K_DW_CL:
        // The ring kernels where they apply; the generic schedule otherwise
        // or when forced (the only selectable dw_cl schedule).
        if (force_variant >= 0 &&
            (force_variant != DWCL_GENERIC || !(dwcl_generic_ok(*d, yb) || dwcl_tgeneric_ok(*d, yb))))
            return CONV_EUNSUPPORTED;
        geom_dwcl(*d, plan, force_variant == DWCL_GENERIC || !dwcl_ring_ok(*d, yb));
        break;
    case CONV_K_PLANE:
        if (!geom_plane(*d, plan)) {
            if (force_kernel != CONV_K_AUTO) return CONV_EUNSUPPORTED;
            plan.kernel = CONV_K_IGEMM;
            if (!geom_igemm(*d, plan, -1)) return CONV_EUNSUPPORTED;
        }
        break;
    case CONV_K_GRP:
        if (!grp_geometry(*d, plan)) return CONV_EUNSUPPORTED;
        if (force_variant >= 0) {
            // The matrix-core schedule only where its own conditions hold.
            if (force_variant == GRP_SCHED_MMA && plan.variant != GRP_SCHED_MMA) return CONV_EUNSUPPORTED;
            if (force_variant > GRP_SCHED_MMA) return CONV_EUNSUPPORTED;
            plan.variant = force_variant;
        }
        break;
    case CONV_K_REDUCE: reduce_geometry(*d, plan); break;
    default:
        if (!geom_igemm(*d, plan, force_variant)) return CONV_EUNSUPPORTED;
        break;
    }
    if (plan.grid[0] > kI32) return CONV_EUNSUPPORTED;

    int64_t ny = numel(yb);
    if (ny == 0) plan.grid[0] = 0;
    int64_t max_off = 0;
    for (const conv_tensor *t : {&d->x, &d->w, &yb})
        for (int i = 0; i < t->rank; ++i)
            if (t->sizes[i] > 0) max_off += (t->sizes[i] - 1) * t->strides[i];
    plan.index64 = max_off > kI32 ? 1 : 0;
    plan.flops = algorithmic_flops(*d);
    plan.bytes = (numel(d->x) + numel(d->w) + (d->has_bias ? d->C_out : 0) + ny) * esize(d->dtype);
    *p = plan;
    return CONV_OK;
}

namespace miconv {

// The plan of n images of a chunked plan's batch: its chunk plan when n is a
// whole chunk, otherwise the same kernel planned for n images (the rule's
// kernel if that one does not take them).
int plan_batch_part(const conv_plan_t &whole, int64_t n, conv_plan_t *out)
{
    if (n == whole.batch_chunk) {
        *out = whole;
        out->d.N = n;
        out->d.x.sizes[0] = n;
        out->y.sizes[0] = n;
        out->batch_chunk = 0;
        return CONV_OK;
    }
    conv_desc d = whole.d;
    conv_tensor y = whole.y;
    d.N = n;
    d.x.sizes[0] = n;
    y.sizes[0] = n;
    conv_plan_opts o;
    std::memset(&o, 0, sizeof(o));
    o.force_kernel = whole.kernel;
    o.force_variant = -1;
    if (conv_plan_ex(&d, &y, &o, out) == CONV_OK) return CONV_OK;
    o.force_kernel = CONV_K_AUTO;
    return conv_plan_ex(&d, &y, &o, out);
}

}  // namespace miconv

extern "C" int conv_plan(const conv_desc *d, const conv_tensor *y, int32_t force_kernel, conv_plan_t *p)
{
    conv_plan_opts o;
    std::memset(&o, 0, sizeof(o));
    o.force_kernel = force_kernel;
    o.force_variant = -1;
    return conv_plan_ex(d, y, &o, p);
}
