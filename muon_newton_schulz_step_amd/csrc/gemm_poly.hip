// bf16 polynomial launches: B = bA + cA^2, and the Q A Q products (POLY, POLY_LO).
#include "muon_gemm.h"

namespace muon {

void launch_gemm_poly(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  if (epi == EPI_POLY) launch_gemm_t<bf16_t, EPI_POLY>(tile, a, t, grid, s);
  else launch_gemm_t<bf16_t, EPI_POLY_LO>(tile, a, t, grid, s);
}

}  // namespace muon
