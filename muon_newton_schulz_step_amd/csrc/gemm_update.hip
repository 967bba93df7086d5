// bf16 update launches: X <- aX + BX into the next X state (UPDATE, UPDATE_ROWS).
#include "muon_gemm.h"

namespace muon {

void launch_gemm_update(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  if (epi == EPI_UPDATE) launch_gemm_t<bf16_t, EPI_UPDATE>(tile, a, t, grid, s);
  else launch_gemm_t<bf16_t, EPI_UPDATE_ROWS>(tile, a, t, grid, s);
}

}  // namespace muon
