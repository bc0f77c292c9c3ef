// Part 4 of the fused kernels' variant table.  The table is spread over
// several files only so that its kernels compile in parallel; gemm_kernels.hip
// joins the parts in order.
#include "gemm_fused.hpp"

namespace mxfp4 {

static const Variant kPart[] = {
    V(4, 1, 4, 2, 1), V(4, 1, 4, 2, 2), V(4, 1, 8, 1, 1), V(4, 1, 8, 1, 2), V(4, 2, 1, 1, 1), V(4, 2, 1, 1, 2),
    V(4, 2, 1, 2, 1), V(4, 2, 1, 2, 2), V(4, 2, 1, 4, 1), V(4, 2, 1, 4, 2), V(4, 2, 2, 1, 1), V(4, 2, 2, 1, 2),
    V(4, 2, 2, 2, 1), V(4, 2, 2, 2, 2), V(4, 2, 4, 1, 1), V(4, 2, 4, 1, 2), V(4, 2, 8, 1, 1), V(4, 2, 8, 1, 2),
    VQ(1, 1, 1, 1, 1), VQ(1, 1, 1, 1, 2), VQ(1, 1, 1, 1, 4), VQ(1, 1, 1, 4, 1), VQ(1, 1, 1, 4, 2), VQ(1, 1, 1, 4, 4),
    VQ(1, 1, 1, 8, 1), VQ(1, 1, 1, 8, 2), VQ(1, 1, 1, 8, 4), VQ(1, 1, 1, 16, 1), VQ(1, 1, 1, 16, 2),
    VQ(1, 1, 1, 16, 4), VQ(1, 1, 2, 1, 1), VQ(1, 1, 2, 1, 2), VQ(1, 1, 2, 1, 4), VQ(1, 1, 2, 4, 1), VQ(1, 1, 2, 4, 2),
    VQ(1, 1, 2, 4, 4), VQ(1, 1, 2, 8, 1), VQ(1, 1, 2, 8, 2), VQ(1, 1, 2, 8, 4), VQ(1, 2, 1, 1, 1), VQ(1, 2, 1, 1, 2),
    VQ(1, 2, 1, 1, 4), VQ(1, 2, 1, 4, 1), VQ(1, 2, 1, 4, 2),
};
// (a host function: the device pass compiles the kernels the table names,
// but emits no reference to the host launchers)
const Variant *variants_part4(int *count) {
  *count = (int)(sizeof(kPart) / sizeof(kPart[0]));
  return kPart;
}

}  // namespace mxfp4
