// Part 0 of the fused kernels' variant table.  The table is spread over
// several files only so that its kernels compile in parallel; gemm_kernels.hip
// joins the parts in order.
#include "gemm_fused.hpp"

namespace mxfp4 {

static const Variant kPart[] = {
    MXFP4_WIDE_VARIANTS(VW) MXFP4_WIDEL_VARIANTS(VWL) VE(1, 2, 1, 8, 4, 16) VE(1, 1, 4, 4, 4, 16)
    VE(1, 2, 1, 8, 2, 16) VE(1, 1, 1, 8, 4, 16) VE(1, 2, 1, 4, 4, 16) VE(1, 1, 2, 4, 4, 16) VE(1, 2, 4, 4, 4, 16)
    VE(1, 2, 1, 8, 4, 8) VE(1, 1, 1, 8, 4, 8) VE(1, 1, 4, 4, 4, 8) V8(1, 1, 1, 16, 4), V8(1, 1, 1, 14, 4),
    V8(1, 1, 1, 8, 4), V8(1, 1, 1, 16, 2), V8(1, 1, 2, 8, 4), V8(1, 1, 2, 8, 2), V8(1, 2, 1, 16, 4),
    V8(1, 2, 1, 8, 4), V8(1, 1, 1, 4, 4), V8(1, 1, 1, 4, 2), V8(1, 1, 1, 8, 2), V8(1, 1, 1, 4, 1), V8(1, 1, 2, 4, 2),
    V8(1, 1, 4, 4, 4), V8(1, 1, 1, 2, 2), V8(1, 1, 1, 1, 4), V8(1, 1, 1, 2, 4), V(1, 2, 1, 12, 1), V(1, 2, 1, 6, 2),
    V(1, 2, 1, 4, 3), V(1, 2, 1, 3, 4), V(1, 1, 1, 12, 1), V(1, 1, 1, 6, 2), V(1, 1, 2, 6, 2),
};
// (a host function: the device pass compiles the kernels the table names,
// but emits no reference to the host launchers)
const Variant *variants_part0(int *count) {
  *count = (int)(sizeof(kPart) / sizeof(kPart[0]));
  return kPart;
}

}  // namespace mxfp4
