// Part 7 of the fused kernels' variant table.  The table is spread over
// several files only so that its kernels compile in parallel; gemm_kernels.hip
// joins the parts in order.
#include "gemm_fused.hpp"

namespace mxfp4 {

static const Variant kPart[] = {
    // 16 x 112 tiles (7 subtiles per wave, odd column groups on every other
    // tile): exactly 256 workgroups at N = 7168
    V(1, 7, 1, 2, 8), V(1, 7, 1, 4, 4), V(1, 7, 1, 8, 2), V(1, 7, 1, 16, 1), V(1, 1, 7, 2, 8), V(1, 1, 7, 1, 16),
    // 32 x 96 tiles: 256 workgroups at M = 256, N = 3072; 12 K steps covered exactly
    V(2, 6, 1, 4, 3), V(2, 6, 1, 6, 2), V(2, 6, 1, 2, 6), V(2, 3, 2, 4, 3), V(2, 3, 2, 2, 6), V(2, 3, 2, 6, 2),
    V(2, 3, 2, 3, 4), V(2, 2, 3, 4, 3), V(2, 2, 3, 2, 6), V(2, 2, 3, 3, 4), V(2, 1, 6, 2, 6),
    VQ(4, 2, 2, 1, 4), VQ(4, 2, 2, 2, 1), VQ(4, 2, 2, 2, 2), VQ(4, 2, 2, 2, 4), VQ(4, 2, 4, 1, 1), VQ(4, 2, 4, 1, 2),
    VQ(4, 2, 4, 1, 4), VQ(4, 4, 1, 1, 1), VQ(4, 4, 1, 1, 2), VQ(4, 4, 1, 1, 4), VQ(4, 4, 1, 2, 1), VQ(4, 4, 1, 2, 2),
    VQ(4, 4, 1, 2, 4), VQ(4, 4, 2, 1, 1), VQ(4, 4, 2, 1, 2), VQ(4, 4, 2, 1, 4), VQ(4, 4, 4, 1, 1), VQ(4, 4, 4, 1, 2),
    VQ(4, 4, 4, 1, 4), VQ(8, 1, 1, 1, 1), VQ(8, 1, 1, 1, 2), VQ(8, 1, 1, 1, 4), VQ(8, 1, 1, 2, 1), VQ(8, 1, 1, 2, 2),
    VQ(8, 1, 1, 2, 4), VQ(8, 1, 1, 4, 1), VQ(8, 1, 1, 4, 2), VQ(8, 1, 1, 4, 4), VQ(8, 1, 2, 1, 1), VQ(8, 1, 2, 1, 2),
    VQ(8, 1, 2, 1, 4), VQ(8, 1, 2, 2, 1), VQ(8, 1, 2, 2, 2), VQ(8, 1, 2, 2, 4), VQ(8, 2, 1, 1, 1), VQ(8, 2, 1, 1, 2),
    VQ(8, 2, 1, 1, 4), VQ(8, 2, 1, 2, 1), VQ(8, 2, 1, 2, 2), VQ(8, 2, 1, 2, 4), VQ(8, 2, 2, 1, 1), VQ(8, 2, 2, 1, 2),
    VQ(8, 2, 2, 1, 4),
    // pre-quantized A, long K at M <= 16 without a K split: 8 waves of 8
    // steps (K up to 8192), faster at K 7168 than 16 waves of 4 (no
    // quantization to spread over the waves)
    VQ(1, 1, 1, 8, 8),
};
// (a host function: the device pass compiles the kernels the table names,
// but emits no reference to the host launchers)
const Variant *variants_part7(int *count) {
  *count = (int)(sizeof(kPart) / sizeof(kPart[0]));
  return kPart;
}

}  // namespace mxfp4
