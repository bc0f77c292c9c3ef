// Part 2 of the fused kernels' variant table.  The table is spread over
// several files only so that its kernels compile in parallel; gemm_kernels.hip
// joins the parts in order.
#include "gemm_fused.hpp"

namespace mxfp4 {

static const Variant kPart[] = {
    V(1, 2, 1, 1, 4), V(1, 2, 1, 2, 1), V(1, 2, 1, 2, 2), V(1, 2, 1, 2, 4), V(1, 2, 1, 4, 1), V(1, 2, 1, 4, 2),
    V(1, 2, 1, 4, 4), V(1, 2, 1, 8, 1), V(1, 2, 1, 8, 2), V(1, 2, 1, 8, 4), V(1, 2, 1, 16, 1), V(1, 2, 1, 16, 2),
    V(1, 2, 2, 1, 1), V(1, 2, 2, 1, 2), V(1, 2, 2, 1, 4), V(1, 2, 2, 2, 1), V(1, 2, 2, 2, 2), V(1, 2, 2, 2, 4),
    V(1, 2, 2, 4, 1), V(1, 2, 2, 4, 2), V(1, 2, 2, 4, 4), V(1, 2, 2, 8, 1), V(1, 2, 2, 8, 2), V(1, 2, 2, 8, 4),
    V(1, 2, 4, 1, 1), V(1, 2, 4, 1, 2), V(1, 2, 4, 1, 4), V(1, 2, 4, 2, 1), V(1, 2, 4, 2, 2), V(1, 2, 4, 2, 4),
    V(1, 2, 4, 4, 1), V(1, 2, 4, 4, 2), V(1, 2, 4, 4, 4), V(2, 1, 1, 1, 1), V(2, 1, 1, 1, 2), V(2, 1, 1, 2, 1),
    V(2, 1, 1, 2, 2), V(2, 1, 1, 4, 1), V(2, 1, 1, 4, 2), V(2, 1, 1, 8, 1), V(2, 1, 1, 8, 2), V(2, 1, 2, 1, 1),
    V(2, 1, 2, 1, 2), V(2, 1, 2, 2, 1),
};
// (a host function: the device pass compiles the kernels the table names,
// but emits no reference to the host launchers)
const Variant *variants_part2(int *count) {
  *count = (int)(sizeof(kPart) / sizeof(kPart[0]));
  return kPart;
}

}  // namespace mxfp4
