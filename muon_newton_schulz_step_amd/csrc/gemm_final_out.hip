// bf16 last-step launches into the caller's output, wide and tall (FINAL_OUT, FINAL_OUT_T).
#include "muon_gemm.h"

namespace muon {

void launch_gemm_final_out(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  if (epi == EPI_FINAL_OUT) launch_gemm_t<bf16_t, EPI_FINAL_OUT>(tile, a, t, grid, s);
  else launch_gemm_t<bf16_t, EPI_FINAL_OUT_T>(tile, a, t, grid, s);
}

}  // namespace muon
