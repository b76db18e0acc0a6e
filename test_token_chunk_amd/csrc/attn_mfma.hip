// bf16 attention entry points (interim: route to the SIMT kernels).
#include "kernels.h"
hipError_t swa_fwd_mfma(const AttnArgs& a, hipStream_t s) { return swa_fwd_simt<bf16>(a, s); }
hipError_t swa_bwd_mfma(const AttnBwdArgs& a, hipStream_t s) { return swa_bwd_simt<bf16>(a, s); }
