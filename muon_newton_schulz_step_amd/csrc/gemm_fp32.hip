// fp32 path: every epilogue on 128 x 128 tiles with register-staged loads.
#include "muon_gemm.h"

namespace muon {

void launch_gemm_fp32(int epi, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_GRAM: launch_gemm_t<float, EPI_GRAM>(128, a, t, grid, s); break;
    case EPI_POLY: launch_gemm_t<float, EPI_POLY>(128, a, t, grid, s); break;
    case EPI_UPDATE: launch_gemm_t<float, EPI_UPDATE>(128, a, t, grid, s); break;
    case EPI_FINAL_W: launch_gemm_t<float, EPI_FINAL_W>(128, a, t, grid, s); break;
    case EPI_FINAL_OUT: launch_gemm_t<float, EPI_FINAL_OUT>(128, a, t, grid, s); break;
    case EPI_FINAL_W_T: launch_gemm_t<float, EPI_FINAL_W_T>(128, a, t, grid, s); break;
    default: launch_gemm_t<float, EPI_FINAL_OUT_T>(128, a, t, grid, s); break;
  }
}

}  // namespace muon
