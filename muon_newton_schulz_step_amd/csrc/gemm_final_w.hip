// bf16 last-step launches into the weights, wide and tall (FINAL_W, FINAL_W_T).
#include "muon_gemm.h"

namespace muon {

void launch_gemm_final_w(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  if (epi == EPI_FINAL_W) launch_gemm_t<bf16_t, EPI_FINAL_W>(tile, a, t, grid, s);
  else launch_gemm_t<bf16_t, EPI_FINAL_W_T>(tile, a, t, grid, s);
}

}  // namespace muon
