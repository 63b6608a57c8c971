// The wide int8 verify-window kernel's translation unit (its four instances:
// D 128 or 256, with or without a draft tree).
#include "wide_kernel.h"

namespace selattn {
namespace mk {

hipError_t wide_launch(const MParams& p, dim3 grid, hipStream_t st) {
    if (p.tree) {
        return p.D == 256 ? wide_launch_one<SEL_ATTN_I8, 256, true>(p, grid, st)
                          : wide_launch_one<SEL_ATTN_I8, 128, true>(p, grid, st);
    }
    return p.D == 256 ? wide_launch_one<SEL_ATTN_I8, 256, false>(p, grid, st)
                      : wide_launch_one<SEL_ATTN_I8, 128, false>(p, grid, st);
}

}  // namespace mk
}  // namespace selattn
