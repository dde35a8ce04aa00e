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

// Implicit GEMM schedule table (kernel CONV_K_IGEMM / CONV_K_IGEMM_T).
struct IgemmCfg {
    int bm, bn, bk;     // workgroup tile: rows, columns, K per step
    int wm, wn;         // waves along rows / columns (block = 64 * wm * wn)
    int stages;         // LDS stages of the direct-to-LDS pipeline
    int eff;            // measured relative MFMA throughput of the schedule, percent
};
const IgemmCfg &igemm_cfg(int variant);
int igemm_num_cfgs();

// Plan-field indices for the implicit GEMM (plan.tile[]).
enum { IG_CIG_PAD = 0, IG_COG_PAD = 1, IG_PHASES = 2, IG_MTILES = 3, IG_NTILES = 4, IG_ROWS = 5, IG_XBYTES = 6 };

// Depthwise channels-last stencil (kernel CONV_K_DW_CL): a lane's strip of TO
// outputs reads NCOL input columns per row.  Each wave streams input rows
// through a ring of D rows in LDS (direct-to-LDS loads); before it reads a
// ring row it waits until at most the VMEM instructions issued after that
// row's loads are pending: D-1 rows of loads plus the stores of D-1 steps
// (every S-th step completes an output row).  With q (the wave's 64 lanes are
// 64 consecutive channel words of one strip) a row takes ceil(NCOL/4)
// 16-byte loads and an output row ceil(TO/4) 16-byte stores; otherwise NCOL
// and TO 4-byte ones.  D is the deepest ring (up to 4) whose worst case fits
// the 6-bit vmcnt field.
constexpr int dwcl_ncol(int K, int S, int TO) { return (TO - 1) * S + K; }
constexpr int dwcl_loads_per_row(int K, int S, int TO, bool q)
{
    return q ? (dwcl_ncol(K, S, TO) + 3) / 4 : dwcl_ncol(K, S, TO);
}
constexpr int dwcl_stores_per_row(int TO, bool q) { return q ? (TO + 3) / 4 : TO; }
constexpr int dwcl_ring_cols(int K, int S, int TO, bool q) { return q ? 4 * dwcl_loads_per_row(K, S, TO, q) : dwcl_ncol(K, S, TO); }
constexpr int dwcl_pending(int K, int S, int TO, int D, bool q)
{
    return (D - 1) * dwcl_loads_per_row(K, S, TO, q) + ((D - 1 + S - 1) / S) * dwcl_stores_per_row(TO, q);
}
constexpr int dwcl_ring_depth(int K, int S, int TO, bool q)
{
    return dwcl_pending(K, S, TO, 4, q) <= 63 ? 4 : dwcl_pending(K, S, TO, 3, q) <= 63 ? 3 : 2;
}

// Launchers (defined in the .hip files).  `vec` selects the 16-byte path.
int launch_igemm(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *ws,
                 void *stream, bool vec);
int launch_plane(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream);
int launch_dwcl(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream,
                bool vec);
int launch_grp(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream);
int launch_reduce(const conv_plan_t &p, const void *x, const void *w, const void *b, void *y, void *stream);

}  // namespace miconv
