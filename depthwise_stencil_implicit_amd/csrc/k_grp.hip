// Few-channel grouped stencil with packed dot2 (kernel CONV_K_GRP).
// Not yet built: the planner routes grouped calls to CONV_K_PLANE meanwhile.
#include "dev_common.h"
#include "internal.h"

namespace miconv {

bool grp_supported(const conv_desc &) { return false; }

void grp_geometry(const conv_desc &, conv_plan_t &p) { p.grid[0] = 0; }

int launch_grp(const conv_plan_t &, const void *, const void *, const void *, void *, void *)
{
    return CONV_EUNSUPPORTED;
}

}  // namespace miconv
