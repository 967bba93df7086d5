// bf16 Gram launches: A = X X^T on lower-triangle tiles (GRAM, GRAM_LO).
#include "muon_gemm.h"

namespace muon {

void launch_gemm_gram(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  if (epi == EPI_GRAM) launch_gemm_t<bf16_t, EPI_GRAM>(tile, a, t, grid, s);
  else launch_gemm_t<bf16_t, EPI_GRAM_LO>(tile, a, t, grid, s);
}

}  // namespace muon
