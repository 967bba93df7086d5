// bf16 last-step launches into the weights: wide, tall, or both kinds in one
// launch (FINAL_W, FINAL_W_T, FINAL_W_MIX).
#include "muon_gemm.h"

namespace muon {

void launch_gemm_final_w(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  if (epi == EPI_FINAL_W) launch_gemm_t<bf16_t, EPI_FINAL_W>(tile, a, t, grid, s);
  else if (epi == EPI_FINAL_W_T) launch_gemm_t<bf16_t, EPI_FINAL_W_T>(tile, a, t, grid, s);
  else launch_gemm_t<bf16_t, EPI_FINAL_W_MIX>(tile, a, t, grid, s);
}

}  // namespace muon
