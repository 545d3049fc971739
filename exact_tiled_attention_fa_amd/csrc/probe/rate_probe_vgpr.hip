// The instruction-rate probes with every MFMA's accumulator and result in
// ArchVGPRs: this file is compiled with -mllvm -amdgpu-mfma-vgpr-form.
#define FA_PROBE_RATES_NAME fa_probe_rates_vgpr
#include "rate_probe.hip"
