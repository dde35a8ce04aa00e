// conv_run: check the call and enqueue the planned kernel(s) on the caller's
// stream; plus the name/status helpers of the C ABI.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <mutex>

#include <algorithm>
#include <cstring>

#include "internal.h"

namespace {

using namespace miconv;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t numel(const conv_tensor &t)
{
    int64_t n = 1;
    for (int i = 0; i < t.rank; ++i) n *= t.sizes[i];
    return n;
}

// Whether the process sees a GPU: asked once, on the first launch.
bool have_device()
{
    static std::once_flag once;
    static bool ok = false;
    std::call_once(once, [] {
        int n = 0;
        ok = hipGetDeviceCount(&n) == hipSuccess && n > 0;
        if (!ok) (void)hipGetLastError();
    });
    return ok;
}

}  // namespace

extern "C" int conv_run(const conv_plan_t *p, const void *x, const void *w, const void *b, void *y,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    if (!p) return CONV_EINVAL;
    const conv_desc &d = p->d;
    if (numel(p->y) == 0 || p->grid[0] == 0) return CONV_OK;
    if (!x || !w || !y) return CONV_EINVAL;
    if (d.has_bias != (b != nullptr)) return CONV_EINVAL;
    const uintptr_t es = (uintptr_t)esize(d.dtype);
    if (!aligned(x, es) || !aligned(w, es) || !aligned(y, es) || (b && !aligned(b, es))) return CONV_EALIGN;
    if (p->workspace_bytes > 0) {
        if (!workspace || workspace_bytes < (size_t)p->workspace_bytes) return CONV_EINVAL;
        if (!aligned(workspace, 16)) return CONV_EALIGN;
    }
    if (!have_device()) return CONV_EDEVICE;
    if (p->batch_chunk > 0 && p->batch_chunk < d.N) {
        // x or y spans 2 GiB or more: the batch in chunks of images, each a
        // plain call on its own slices of x and y.
        const int64_t xs = d.x.strides[0] * (int64_t)es, ys = p->y.strides[0] * (int64_t)es;
        for (int64_t n0 = 0; n0 < d.N; n0 += p->batch_chunk) {
            conv_plan_t sub;
            int st = plan_batch_part(*p, std::min<int64_t>(p->batch_chunk, d.N - n0), &sub);
            if (st != CONV_OK) return st;
            if (sub.workspace_bytes > p->workspace_bytes) return CONV_EINVAL;
            st = conv_run(&sub, static_cast<const char *>(x) + n0 * xs, w, b, static_cast<char *>(y) + n0 * ys,
                          workspace, workspace_bytes, stream);
            if (st != CONV_OK) return st;
        }
        return CONV_OK;
    }
    const bool vec = p->vec_ok && aligned(x, 16) && aligned(y, 16);
    switch (p->kernel) {
    case CONV_K_DW_CL:
        // Lanes move 4-byte channel words; a view that is not word-aligned
        // runs on the layout-generic plane stencil instead (the transposed
        // schedule moves single elements).
        if (!d.transposed && (!aligned(x, 4) || !aligned(y, 4))) {
            conv_tensor yc = p->y;
            if (d.unbatched) {
                for (int i = 1; i < yc.rank; ++i) {
                    yc.sizes[i - 1] = yc.sizes[i];
                    yc.strides[i - 1] = yc.strides[i];
                }
                yc.rank -= 1;
            }
            conv_plan_t q;
            const int st = conv_plan(&d, &yc, CONV_K_PLANE, &q);
            if (st != CONV_OK) return st;
            return launch_plane(q, x, w, b, y, stream);
        }
        return launch_dwcl(*p, x, w, b, y, stream, vec);
    case CONV_K_PLANE: return launch_plane(*p, x, w, b, y, stream);
    case CONV_K_GRP: return launch_grp(*p, x, w, b, y, stream);
    case CONV_K_REDUCE: return launch_reduce(*p, x, w, b, y, stream);
    case CONV_K_IGEMM_T:
        // The both-phases tile loads x in 16-byte chunks.  An x view off a
        // 16-byte boundary runs on the phase-split tile of 64 output channels
        // (configuration 3), whose repacked weights have the same layout and
        // size, so the plan's workspace serves it.
        if ((p->variant == IG_T1_CFG || p->variant == IG_T1B_CFG) && !aligned(x, 16)) {
            conv_tensor yc = p->y;
            if (d.unbatched) {
                for (int i = 1; i < yc.rank; ++i) {
                    yc.sizes[i - 1] = yc.sizes[i];
                    yc.strides[i - 1] = yc.strides[i];
                }
                yc.rank -= 1;
            }
            conv_plan_opts o;
            std::memset(&o, 0, sizeof(o));
            o.force_kernel = CONV_K_IGEMM_T;
            o.force_variant = 3;
            conv_plan_t q;
            const int st = conv_plan_ex(&d, &yc, &o, &q);
            if (st != CONV_OK) return st;
            if (q.workspace_bytes > p->workspace_bytes) return CONV_EALIGN;
            return launch_igemm(q, x, w, b, y, workspace, stream, false);
        }
        return launch_igemm(*p, x, w, b, y, workspace, stream, vec);
    case CONV_K_IGEMM: return launch_igemm(*p, x, w, b, y, workspace, stream, vec);
    default: return CONV_EINVAL;
    }
}

extern "C" const char *conv_kernel_name(int32_t kernel)
{
    switch (kernel) {
    case CONV_K_AUTO: return "auto";
    case CONV_K_DW_CL: return "dw_cl";
    case CONV_K_PLANE: return "plane";
    case CONV_K_GRP: return "grp";
    case CONV_K_REDUCE: return "reduce";
    case CONV_K_IGEMM: return "igemm";
    case CONV_K_IGEMM_T: return "igemm_t";
    default: return "?";
    }
}

extern "C" const char *conv_status_string(int32_t status)
{
    switch (status) {
    case CONV_OK: return "ok";
    case CONV_EINVAL: return "invalid argument";
    case CONV_EUNSUPPORTED: return "kernel does not support this call";
    case CONV_ELAYOUT: return "output layout differs from conv_out_shape";
    case CONV_EALIGN: return "pointer not aligned to its element size";
    case CONV_EDEVICE: return "no usable GPU or HIP launch error";
    case CONV_ENOSPACE: return "the plan needs more scratch than conv_run_noalloc's fixed device array holds";
    default: return "unknown status";
    }
}

extern "C" int32_t conv_abi_version(void) { return 3; }
