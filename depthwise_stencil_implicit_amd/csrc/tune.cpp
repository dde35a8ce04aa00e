// conv_plan_candidates / conv_tune / conv_plan_tuned: plan-time timing of the
// schedules that can run a call, with the fastest cached per descriptor.
//
// executorch PR #25085 ("Route 2-D depthwise and few-channel grouped
// convolutions to a Triton direct-stencil kernel"), description: the
// stencil's schedules are timed when the call is compiled and the fastest
// is kept; torch/_inductor/kernel/conv.py (the convolution lowering) picks
// among its templates with autotune_select_algorithm.  Here the candidates
// are the plans conv_plan_ex accepts for the call -- every kernel whose
// supports() holds, and every schedule of the kernels that have several --
// timed on the caller's own buffers and stream.
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "internal.h"

namespace {

using namespace miconv;

std::mutex g_mu;
std::map<std::string, conv_plan_t> g_cache;   // (descriptor, y, device) -> fastest plan

std::string key_of(const conv_desc &d, const conv_tensor &y, int dev)
{
    std::string k(reinterpret_cast<const char *>(&d), sizeof(d));
    k.append(reinterpret_cast<const char *>(&y), sizeof(y));
    k.append(reinterpret_cast<const char *>(&dev), sizeof(dev));
    return k;
}

int add(const conv_desc *d, const conv_tensor *y, int32_t kernel, int32_t variant, conv_plan_t *out, int32_t max,
        int32_t &n)
{
    conv_plan_opts o;
    std::memset(&o, 0, sizeof(o));
    o.force_kernel = kernel;
    o.force_variant = variant;
    conv_plan_t p;
    if (conv_plan_ex(d, y, &o, &p) != CONV_OK) return 0;
    // An implicit GEMM that pads each group's input channels more than
    // fourfold to its channel block (a depthwise or few-channel call, which
    // the stencils serve) multiplies mostly zeros: one launch can take
    // milliseconds, so it is not timed.
    if ((p.kernel == CONV_K_IGEMM || p.kernel == CONV_K_IGEMM_T) && !(p.flags & CONV_PLAN_ONE_BY_ONE) &&
        p.tile[IG_CIG_PAD] > 4 * (d->C_in / d->groups))
        return 0;
    // The same schedule reached through another forced kernel (a plane plan
    // can fall back to the implicit GEMM) is listed once.
    for (int i = 0; i < n && i < max; ++i)
        if (out[i].kernel == p.kernel && out[i].variant == p.variant && out[i].flags == p.flags) return 0;
    if (n < max) out[n] = p;
    ++n;
    return 1;
}

}  // namespace

extern "C" int conv_plan_candidates(const conv_desc *d, const conv_tensor *y, conv_plan_t *out, int32_t max,
                                    int32_t *count)
{
    if (!d || !y || !count || (max > 0 && !out)) return CONV_EINVAL;
    conv_plan_t probe;
    const int st = conv_plan(d, y, CONV_K_AUTO, &probe);
    if (st != CONV_OK) return st;
    int32_t n = 0;
    // The rule's own plan first.
    if (max > 0) out[0] = probe;
    n = 1;
    for (int32_t k : {CONV_K_DW_CL, CONV_K_PLANE}) add(d, y, k, -1, out, max, n);
    // The generic channels-last schedule only where no ring schedule applies:
    // it re-reads each input row once per kernel row from L2, which timing
    // on the caller's (warm) buffers rewards and a cold input does not (3x3
    // stride 2: 14.7 us on the ring, 20.5 us generic, with the input out of
    // the caches).
    const bool ring = probe.kernel == CONV_K_DW_CL && probe.variant != DWCL_GENERIC;
    if (!ring) add(d, y, CONV_K_DW_CL, DWCL_GENERIC, out, max, n);
    // The one-wave-per-output reduction only where outputs are few.
    if (d->out[0] * d->out[1] * d->out[2] <= 16) add(d, y, CONV_K_REDUCE, -1, out, max, n);
    for (int32_t v : {GRP_SCHED_VALU, GRP_SCHED_MMA}) add(d, y, CONV_K_GRP, v, out, max, n);
    const int32_t gk = d->transposed ? CONV_K_IGEMM_T : CONV_K_IGEMM;
    for (int32_t v = 0; v < igemm_num_cfgs(); ++v)
        if (v != IG_TAIL_CFG) add(d, y, gk, v, out, max, n);
    if (d->transposed) {
        add(d, y, gk, IG_T1_CFG, out, max, n);
        add(d, y, gk, IG_T1B_CFG, out, max, n);
    }
    *count = n;
    return CONV_OK;
}

extern "C" int conv_tune(const conv_desc *d, const conv_tensor *y, const void *x, const void *w, const void *b,
                         void *yptr, void *workspace, size_t workspace_bytes, void *stream, int32_t reps,
                         conv_plan_t *best)
{
    if (!d || !y || !best) return CONV_EINVAL;
    constexpr int32_t kMax = 64;
    conv_plan_t cand[kMax];
    int32_t n = 0;
    int st = conv_plan_candidates(d, y, cand, kMax, &n);
    if (st != CONV_OK) return st;
    if (n > kMax) n = kMax;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return CONV_EDEVICE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return CONV_EDEVICE;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return CONV_EDEVICE;
    }
    if (reps < 1) reps = 1;
    int chosen = -1;
    float best_ms = 0.f;
    for (int i = 0; i < n; ++i) {
        const conv_plan_t &p = cand[i];
        if ((size_t)p.workspace_bytes > workspace_bytes) continue;   // does not fit the caller's workspace
        // One untimed launch (code-object load, caches), then reps timed ones.
        if (conv_run(&p, x, w, b, yptr, workspace, workspace_bytes, stream) != CONV_OK) continue;
        if (hipEventRecord(e0, s) != hipSuccess) break;
        bool ok = true;
        for (int r = 0; r < reps && ok; ++r) ok = conv_run(&p, x, w, b, yptr, workspace, workspace_bytes, stream) == CONV_OK;
        if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) break;
        float ms = 0.f;
        if (!ok || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) continue;
        if (chosen < 0 || ms < best_ms) {
            chosen = i;
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipGetLastError();
    if (chosen < 0) return CONV_EDEVICE;
    *best = cand[chosen];
    std::lock_guard<std::mutex> lock(g_mu);
    g_cache[key_of(*d, *y, dev)] = cand[chosen];
    return CONV_OK;
}

extern "C" int conv_plan_tuned(const conv_desc *d, const conv_tensor *y, conv_plan_t *p)
{
    if (!d || !y || !p) return CONV_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = -1;
    }
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_cache.find(key_of(*d, *y, dev));
        if (it != g_cache.end()) {
            *p = it->second;
            p->flags |= CONV_PLAN_TUNED;
            return CONV_OK;
        }
    }
    return conv_plan(d, y, CONV_K_AUTO, p);
}
