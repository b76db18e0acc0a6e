// bf16 GEMM entry point (interim: routes to the SIMT kernel).
#include "kernels.h"
hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s) { return gemm_simt_bf16(g, s); }
