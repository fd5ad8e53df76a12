// The fused GEMM pair kernels: a layer's dX (NN) and dW (TN) in one launch,
// on the 128x128 and 64x64 unit tiles, all four format pairs.
#include "gemm_kernel.h"

namespace fp8ds {

namespace {

GemmPairFn pick_pair_u128s(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_pair_u128s_kernel<true, false, false, false, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_pair_u128s_kernel<true, false, false, false, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_pair_u128s_kernel<true, false, false, false, 0, 1>;
  return gemm_pair_u128s_kernel<true, false, false, false, 1, 1>;
}

GemmPairFn pick_pair_u128t(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_pair_u128t_kernel<true, false, false, false, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_pair_u128t_kernel<true, false, false, false, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_pair_u128t_kernel<true, false, false, false, 0, 1>;
  return gemm_pair_u128t_kernel<true, false, false, false, 1, 1>;
}

}  // namespace

GemmPairFn gemm_pair_fn(int tile, int fa, int fb) {
  return tile == 8 ? pick_pair_u128t(fa, fb) : pick_pair_u128s(fa, fb);
}

}  // namespace fp8ds
