// conv_backward_layout / conv_plan_backward / conv_run_backward: the
// gradients of the canonical op (torch/_inductor/kernel/conv.py,
// convolution_backward: input, weight and bias gradients of one call).
//
// Input gradient.  The op is linear in x, and its adjoint in x is the same
// call with forward and transposed exchanged, on the same weight tensor: a
// forward call's dx is the transposed call of gy (weight [C_out, Cig, k]
// read as [C_in', Cog', k]) with output_padding (L + pb + pa - dil(k-1) - 1)
// mod s, whose output length is exactly L; a transposed call's dx is the
// forward call of gy (output length L as long as output_padding < stride).
// So dx runs on the planner's own kernels, chosen for that call.  With stride
// 1 the transposed adjoint is itself a forward call: per dim
//   dx[i] = sum_t gy[i + pb - t*dil] w[t] = sum_t' gy[i - pb' + t'*dil] w[K-1-t']
// with pb' = (K-1)*dil - pb, a correlation of gy with the taps reversed and,
// per group, the two channel dims of the weight exchanged.  Where that forward
// call has at most 8 input channels per group (depthwise and few-channel
// grouped calls, whose transposed adjoint the implicit GEMM would pad to its
// 64-channel K step), the weight is first copied reversed into the workspace
// and dx runs on the forward stencils.
//
// Weight and bias gradients.  The weight gradient is the GEMM over
// positions described in k_bwd.hip, split over workgroups by ranges of
// positions with fp32 partial sums that a reduction adds and rounds once; the
// bias gradient sums gy per channel the same way.
#include <cstring>
#include <algorithm>

#include "internal.h"

namespace {

using namespace miconv;

constexpr int64_t kI32 = 0x7fffffffLL;

int64_t numel(const conv_tensor &t)
{
    int64_t n = 1;
    for (int i = 0; i < t.rank; ++i) n *= t.sizes[i];
    return n;
}

int64_t span_bytes(const conv_tensor &t, int64_t es)
{
    int64_t off = 0;
    for (int i = 0; i < t.rank; ++i)
        if (t.sizes[i] > 0) off += (t.sizes[i] - 1) * t.strides[i];
    return (off + 1) * es;
}

// The batched view of a descriptor of y's shape (unbatched calls add N = 1).
bool batched_like_y(const conv_desc &d, const conv_tensor &in, conv_tensor &out)
{
    conv_tensor yb;
    batched_out(d, yb);
    std::memset(&out, 0, sizeof(out));
    if (in.dtype != d.dtype) return false;
    if (in.rank == yb.rank) {
        out = in;
    } else if (d.unbatched && in.rank == yb.rank - 1) {
        out.rank = yb.rank;
        out.dtype = in.dtype;
        out.sizes[0] = 1;
        out.strides[0] = 0;
        for (int i = 0; i < in.rank; ++i) {
            out.sizes[i + 1] = in.sizes[i];
            out.strides[i + 1] = in.strides[i];
        }
        int64_t ext = 1;
        for (int i = 0; i < in.rank; ++i) ext = std::max(ext, in.strides[i] * std::max<int64_t>(in.sizes[i], 1));
        out.strides[0] = ext;
    } else {
        return false;
    }
    for (int i = 0; i < yb.rank; ++i)
        if (out.sizes[i] != yb.sizes[i] || out.strides[i] < 0) return false;
    return true;
}

// The adjoint call in x: forward <-> transposed on gy with the same weight.
bool adjoint_desc(const conv_desc &d, const conv_tensor &gy, conv_desc &a)
{
    std::memset(&a, 0, sizeof(a));
    a.spatial = d.spatial;
    a.transposed = d.transposed ? 0 : 1;
    a.unbatched = 0;
    a.dtype = d.dtype;
    a.has_bias = 0;
    a.N = d.N;
    a.C_in = d.C_out;
    a.C_out = d.C_in;
    a.groups = d.groups;
    for (int i = 0; i < 3; ++i) {
        a.in[i] = d.out[i];
        a.k[i] = d.k[i];
        a.stride[i] = d.stride[i];
        a.padding_before[i] = d.padding_before[i];
        a.padding_after[i] = d.padding_after[i];
        a.dilation[i] = d.dilation[i];
        a.output_padding[i] = 0;
        if (i >= d.spatial) {
            a.out[i] = 1;
            continue;
        }
        if (!d.transposed) {
            const int64_t span = d.in[i] + d.padding_before[i] + d.padding_after[i] - d.dilation[i] * (d.k[i] - 1) - 1;
            a.output_padding[i] = span % d.stride[i];
        } else if (d.output_padding[i] >= d.stride[i]) {
            return false;   // the forward adjoint would be longer than x
        }
        a.out[i] = d.in[i];
        if (out_len(a.transposed, a.in[i], a.k[i], a.stride[i], a.padding_before[i], a.padding_after[i],
                    a.dilation[i], a.output_padding[i]) != d.in[i])
            return false;
    }
    a.x = gy;
    a.w = d.w;
    std::memset(&a.b, 0, sizeof(a.b));
    return true;
}

// The stride-1 input gradient as a forward call of gy with the reversed,
// channel-exchanged weight (contiguous [C_in][C_out/groups][k...]).
bool flipped_desc(const conv_desc &d, const conv_tensor &gy, conv_desc &f)
{
    if (d.transposed || d.spatial > 2) return false;
    const int64_t Cog = d.C_out / d.groups;
    if (Cog > 8) return false;
    std::memset(&f, 0, sizeof(f));
    f.spatial = d.spatial;
    f.dtype = d.dtype;
    f.N = d.N;
    f.C_in = d.C_out;
    f.C_out = d.C_in;
    f.groups = d.groups;
    for (int i = 0; i < 3; ++i) {
        f.in[i] = d.out[i];
        f.k[i] = d.k[i];
        f.stride[i] = 1;
        f.dilation[i] = d.dilation[i];
        f.out[i] = d.in[i];
        if (i >= d.spatial) continue;
        const int64_t reach = (d.k[i] - 1) * d.dilation[i];
        if (d.stride[i] != 1 || d.padding_before[i] > reach || d.padding_after[i] > reach) return false;
        f.padding_before[i] = reach - d.padding_before[i];
        f.padding_after[i] = reach - d.padding_after[i];
        if (out_len(0, f.in[i], f.k[i], 1, f.padding_before[i], f.padding_after[i], f.dilation[i], 0) != d.in[i])
            return false;
    }
    f.x = gy;
    f.w.rank = d.spatial + 2;
    f.w.dtype = d.dtype;
    f.w.sizes[0] = d.C_in;
    f.w.sizes[1] = Cog;
    for (int i = 0; i < d.spatial; ++i) f.w.sizes[2 + i] = d.k[i];
    int64_t acc = 1;
    for (int i = f.w.rank - 1; i >= 0; --i) {
        f.w.strides[i] = acc;
        acc *= f.w.sizes[i];
    }
    return true;
}

// A channel-major 16-bit gy of 16 MiB or more beside channels-last x is
// first copied channels-last (one transpose pass), so the input and weight
// gradients read both operands in 16-byte channel chunks (and dx takes x's
// channels-last layout).  Returns the bytes of the copy (0: gy is read as
// given) and the layout the gradients read in G.
int64_t gy_stage(const conv_desc &d, const conv_tensor &gyb, conv_tensor &G)
{
    G = gyb;
    const int64_t bytes = numel(gyb) * esize(d.dtype);
    if (d.dtype == CONV_F32 || d.x.strides[1] != 1 || d.N > 65535 || d.C_out < 64 || d.C_out % 8 != 0 ||
        !bgrad_by_rows(d, gyb) || bytes < (16 << 20) || bytes >= kI32 - 4096 ||
        cdiv(numel(gyb) / (d.N * d.C_out), 64) > 65535)
        return 0;
    channels_last_of(gyb, G);
    return round_up(bytes, 256);
}

// Dense strides in the dim order of t's strides (its memory format).
void dense_like(const conv_tensor &t, conv_tensor &o)
{
    o = t;
    int order[CONV_MAX_RANK];
    for (int i = 0; i < t.rank; ++i) order[i] = i;
    // Innermost first: ascending stride, ties keep the later dim inner.
    std::stable_sort(order, order + t.rank, [&](int p, int q) {
        if (t.strides[p] != t.strides[q]) return t.strides[p] < t.strides[q];
        return p > q;
    });
    int64_t acc = 1;
    for (int i = 0; i < t.rank; ++i) {
        o.strides[order[i]] = acc;
        acc *= std::max<int64_t>(t.sizes[order[i]], 1);
    }
}

}  // namespace

extern "C" int conv_backward_layout(const conv_desc *d, const conv_tensor *gy, conv_tensor *dx, conv_tensor *dw,
                                    conv_tensor *db)
{
    if (!d || !gy) return CONV_EINVAL;
    if (d->spatial < 1 || d->spatial > 3 || d->x.rank != d->spatial + 2) return CONV_EINVAL;
    conv_tensor gyb;
    if (!batched_like_y(*d, *gy, gyb)) return CONV_ELAYOUT;
    if (dx) {
        conv_desc a;
        conv_tensor G;
        gy_stage(*d, gyb, G);
        if (!adjoint_desc(*d, G, a)) return CONV_EUNSUPPORTED;
        conv_tensor xb;
        batched_out(a, xb);
        if (!d->unbatched) {
            *dx = xb;
        } else {
            std::memset(dx, 0, sizeof(*dx));
            dx->rank = xb.rank - 1;
            dx->dtype = xb.dtype;
            for (int i = 1; i < xb.rank; ++i) {
                dx->sizes[i - 1] = xb.sizes[i];
                dx->strides[i - 1] = xb.strides[i];
            }
        }
    }
    if (dw) dense_like(d->w, *dw);
    if (db) {
        std::memset(db, 0, sizeof(*db));
        db->rank = 1;
        db->dtype = d->dtype;
        db->sizes[0] = d->C_out;
        db->strides[0] = 1;
    }
    return CONV_OK;
}

extern "C" int conv_plan_backward(const conv_desc *d, const conv_tensor *gy, int32_t need_dx, int32_t need_dw,
                                  int32_t need_db, conv_bwd_plan_t *p)
{
    if (!d || !gy || !p) return CONV_EINVAL;
    if (d->spatial < 1 || d->spatial > 3 || d->x.rank != d->spatial + 2 || d->groups < 1) return CONV_EINVAL;
    conv_bwd_plan_t plan;
    std::memset(&plan, 0, sizeof(plan));
    plan.d = *d;
    if (!batched_like_y(*d, *gy, plan.gy)) return CONV_ELAYOUT;
    plan.need_dx = need_dx ? 1 : 0;
    plan.need_dw = need_dw ? 1 : 0;
    plan.need_db = need_db ? 1 : 0;
    const int64_t es = esize(d->dtype);
    int64_t ws = 0;
    const int64_t M_y = d->N * d->out[0] * d->out[1] * d->out[2];
    // G: the gy layout the gradient kernels read (a channels-last copy of a
    // large channel-major gy, when staged).
    conv_tensor G;
    const int64_t stage = (need_dx || need_dw) ? gy_stage(*d, plan.gy, G) : (G = plan.gy, 0);

    // ---- input gradient: the adjoint call on the planner's kernels ----
    if (plan.need_dx) {
        conv_desc a;
        if (!adjoint_desc(*d, G, a)) return CONV_EUNSUPPORTED;
        batched_out(a, plan.dx);
        conv_desc f;
        conv_plan_t fp;
        if (flipped_desc(*d, G, f) && conv_plan(&f, &plan.dx, CONV_K_AUTO, &fp) == CONV_OK &&
            fp.kernel != CONV_K_IGEMM && fp.kernel != CONV_K_IGEMM_T) {
            // The reversed weight first, then the stencil's own scratch.
            plan.dgrad = fp;
            plan.dgrad_flip = 1;
            ws = std::max<int64_t>(ws, round_up(numel(f.w) * es, 256) + round_up(fp.workspace_bytes, 256));
        } else {
            const int st = conv_plan(&a, &plan.dx, CONV_K_AUTO, &plan.dgrad);
            if (st != CONV_OK) return st;
            ws = std::max<int64_t>(ws, round_up(plan.dgrad.workspace_bytes, 256));
        }
        plan.flops[0] = plan.dgrad.flops;
        plan.bytes[0] = plan.dgrad.bytes;
    }

    // ---- weight gradient ----
    conv_backward_layout(d, gy, nullptr, &plan.dw, nullptr);
    if (plan.need_dw) {
        const bool tr = d->transposed != 0;
        const conv_tensor &P = tr ? d->x : G;
        const conv_tensor &Q = tr ? G : d->x;
        const int64_t Cig = d->C_in / d->groups, Cog = d->C_out / d->groups;
        const int64_t PC = tr ? Cig : Cog, QC = tr ? Cog : Cig;
        const int64_t T = d->k[0] * d->k[1] * d->k[2];
        const int64_t M = tr ? d->N * d->in[0] * d->in[1] * d->in[2] : M_y;
        // Each operand of the matrix-core kernel is read channel-major (16-byte
        // chunks of 8 channels: channel stride 1, the other strides and the
        // channel count multiples of 8, a span below 2 GiB) or position-major
        // (8 positions of one channel element by element: the last spatial
        // extent of the positions a multiple of 8).  Channel counts of at least
        // 32 keep the 128-wide tiles from being mostly padding.
        auto channel_major = [&](const conv_tensor &t, int64_t C) {
            bool ok = t.strides[1] == 1 && C % 8 == 0 && span_bytes(t, es) < kI32 - 4096;
            for (int i = 0; i < t.rank && ok; ++i) ok = i == 1 || t.strides[i] % 8 == 0;
            return ok;
        };
        const int64_t Elast = tr ? d->in[d->spatial - 1] : d->out[d->spatial - 1];
        const bool cm_p = channel_major(P, PC), cm_q = channel_major(Q, QC);
        const bool pm_ok = Elast % 8 == 0;
        bool mfma = d->dtype != CONV_F32 && PC >= 32 && QC >= 32 && (cm_p || pm_ok) && (cm_q || pm_ok);
        // Depthwise on channels-last 16-bit operands: the stencil over channel
        // words (every stride of both operands even, so words stay aligned).
        auto words = [&](const conv_tensor &t) {
            bool ok = t.strides[1] == 1 && span_bytes(t, es) < kI32 - 4096;
            for (int i = 0; i < t.rank && ok; ++i) ok = i == 1 || t.strides[i] % 2 == 0;
            return ok;
        };
        const bool dwk = !tr && d->dtype != CONV_F32 && d->spatial <= 2 && PC == 1 && QC == 1 &&
                         d->groups == d->C_in && d->C_in % 2 == 0 && T <= 88 && words(P) && words(Q);
        if (dwk) mfma = false;
        // Few channels per group on channel-major operands (every (image,
        // channel) plane dense): the plane-staged schedule, one thread per
        // (out channel, in channel, tap), the planes within 64 KB of LDS.
        auto planes = [&](const conv_tensor &t, const int64_t *ext) {
            int64_t acc = 1;
            for (int i = d->spatial - 1; i >= 0; --i) {
                if (ext[i] > 1 && t.strides[2 + i] != acc) return false;
                acc *= ext[i];
            }
            return t.strides[1] != 1 || d->C_in == 1;
        };
        const bool plk = !tr && !dwk && !mfma && d->spatial <= 2 && PC * QC * T <= 1024 &&
                         wgrad_plane_lds(*d) <= 64 * 1024 && planes(P, d->out) && planes(Q, d->in);
        const int64_t mode = dwk ? WB_DW : plk ? WB_PLANE : mfma ? (1 | (cm_p ? 0 : 2) | (cm_q ? 0 : 4)) : 0;
        const int64_t apad = mfma ? round_up(PC, 128) : PC, bpad = mfma ? round_up(QC, 128) : QC;
        const int64_t steps = std::max<int64_t>(1, cdiv(M, 32));
        int64_t splits;
        if (plk) {
            // Ranges of images, about 1024 workgroups.
            splits = std::max<int64_t>(1, std::min<int64_t>(d->N, cdiv(1024, d->groups)));
        } else if (dwk) {
            // Ranges of rows (image, output row), about 1024 workgroups.
            const int64_t rows = d->N * (d->spatial == 2 ? d->out[0] : 1);
            const int64_t per_wg = 2 * 256 / wgrad_dw_tg(T);   // channels of a workgroup
            splits = std::max<int64_t>(1, std::min<int64_t>(rows, cdiv(1024, cdiv(d->C_in, per_wg))));
        } else if (mfma) {
            const int64_t tiles = d->groups * T * (apad / 128) * (bpad / 128);
            splits = std::max<int64_t>(1, std::min<int64_t>(steps / 4 > 0 ? steps / 4 : 1, cdiv(1024, tiles)));
        } else {
            const int64_t elems = d->groups * T * PC * QC;
            splits = std::max<int64_t>(1, std::min<int64_t>(steps, cdiv(1 << 19, std::max<int64_t>(elems, 1))));
        }
        plan.wg_tile[WB_MFMA] = mode;
        plan.wg_tile[WB_APAD] = apad;
        plan.wg_tile[WB_BPAD] = bpad;
        plan.wg_tile[WB_SPLITS] = splits;
        plan.wg_tile[WB_PBYTES] = std::min<int64_t>(span_bytes(P, es), kI32 - 4096);
        plan.wg_tile[WB_QBYTES] = std::min<int64_t>(span_bytes(Q, es), kI32 - 4096);
        ws = std::max<int64_t>(ws, round_up(splits * d->groups * T * apad * bpad * 4, 256));
        plan.flops[1] = 2 * T * PC * QC * d->groups * M;   // every (position, tap) pair, as the forward count
        plan.bytes[1] = (numel(d->x) + numel(plan.gy) + numel(d->w)) * es;
    }

    // ---- bias gradient ----
    if (plan.need_db) {
        const int64_t chunks = cdiv(d->C_out, 64);
        plan.db_splits = bgrad_by_rows(*d, plan.gy)
                             ? d->N
                             : std::max<int64_t>(1, std::min<int64_t>(cdiv(1024, chunks), cdiv(M_y, 64)));
        ws = std::max<int64_t>(ws, round_up(plan.db_splits * d->C_out * 4, 256));
        plan.flops[2] = M_y * d->C_out;
        plan.bytes[2] = (numel(plan.gy) + d->C_out) * es;
        plan.db.rank = 1;
        plan.db.dtype = d->dtype;
        plan.db.sizes[0] = d->C_out;
        plan.db.strides[0] = 1;
    }
    plan.wg_tile[WB_GYCL] = stage;
    plan.workspace_bytes = stage + ws;
    *p = plan;
    return CONV_OK;
}

extern "C" int conv_run_backward(const conv_bwd_plan_t *p, const void *x, const void *w, const void *gy, void *dx,
                                 void *dw, void *db, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!p) return CONV_EINVAL;
    const conv_desc &d = p->d;
    // Empty tensors may come with NULL pointers; what must be written must not.
    const bool have_pos = numel(p->gy) > 0;
    if (have_pos && !gy) return CONV_EINVAL;
    if ((p->need_dx && numel(p->dx) > 0 && (!dx || (have_pos && !w))) ||
        (p->need_dw && numel(p->dw) > 0 && (!dw || (have_pos && numel(d.x) > 0 && !x))) ||
        (p->need_db && d.C_out > 0 && !db))
        return CONV_EINVAL;
    if (p->workspace_bytes > 0) {
        if (!workspace || workspace_bytes < (size_t)p->workspace_bytes) return CONV_EINVAL;
        if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return CONV_EALIGN;
    }
    const uintptr_t es = (uintptr_t)esize(d.dtype);
    for (const void *q : {(const void *)x, (const void *)w, gy, (const void *)dx, (const void *)dw, (const void *)db})
        if (q && (reinterpret_cast<uintptr_t>(q) & (es - 1))) return CONV_EALIGN;
    int st = CONV_OK;
    // A staged gy: the channels-last copy first, then the input and weight
    // gradients read it, with the rest of the workspace after it.
    conv_bwd_plan_t staged;
    const conv_bwd_plan_t *const p0 = p;
    const void *const gy0 = gy;
    const int64_t stage = p->wg_tile[WB_GYCL];
    if (stage > 0 && have_pos) {
        st = launch_gy_to_cl(*p, gy, workspace, stream);
        if (st != CONV_OK) return st;
        staged = *p;
        channels_last_of(p->gy, staged.gy);
        gy = workspace;
        workspace = static_cast<char *>(workspace) + stage;
        workspace_bytes -= (size_t)stage;
        p = &staged;
    }
    if (p->need_dx && numel(p->dx) > 0) {
        if (p->dgrad_flip) {
            const size_t off = (size_t)round_up(numel(p->dgrad.d.w) * (int64_t)es, 256);
            st = launch_flip_weight(*p, w, workspace, stream);
            if (st != CONV_OK) return st;
            st = conv_run(&p->dgrad, gy, workspace, nullptr, dx, static_cast<char *>(workspace) + off,
                          workspace_bytes - off, stream);
        } else {
            st = conv_run(&p->dgrad, gy, w, nullptr, dx, workspace, workspace_bytes, stream);
        }
        if (st != CONV_OK) return st;
    }
    if (p->need_dw && numel(p->dw) > 0) {
        if (!have_pos || numel(d.x) == 0) {
            // No terms: the gradient is zero.
            st = launch_fill_zero(dw, p->dw, stream);
        } else {
            // 16-byte loads (4-byte words for the depthwise stencil) need
            // aligned operands; otherwise the simple kernel.
            conv_bwd_plan_t q = *p;
            const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(gy);
            const int64_t md = q.wg_tile[WB_MFMA];
            if ((md == WB_DW && (al & 3)) ||
                (md != WB_DW && md != WB_PLANE && (md & 6) != 6 && md && (al & 15))) {
                q.wg_tile[WB_MFMA] = 0;
                q.wg_tile[WB_APAD] = d.transposed ? d.C_in / d.groups : d.C_out / d.groups;
                q.wg_tile[WB_BPAD] = d.transposed ? d.C_out / d.groups : d.C_in / d.groups;
            }
            st = launch_wgrad(q, x, gy, dw, workspace, stream);
        }
        if (st != CONV_OK) return st;
    }
    if (p->need_db && d.C_out > 0)
        // The bias gradient reads gy as given (a channel-major gy by rows).
        st = have_pos ? launch_bgrad(*p0, gy0, db, workspace, stream) : launch_fill_zero(db, p->db, stream);
    return st;
}
