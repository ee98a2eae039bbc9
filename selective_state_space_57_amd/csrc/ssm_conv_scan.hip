// The forward scan and the decode step fed through the causal depthwise convolution (+ SiLU) of the Mamba block's SSM
// branch (docs.ifdog.com tutorial, "Mamba 架构" step 3a; Mamba paper section 3.4 for the activation).  Same kernels as
// ssm_scan.hip, instantiated with CONV = true: the lane that owns step t converts x_t, reads x_{t-1..t-3} from its row
// neighbours with DPP row_ror (lanes 0..2 take them from the previous 16-step block, kept in a register; the first
// block of a segment reads them from x or from the incoming convolution state), applies the taps, the bias and SiLU,
// and uses the result wherever the plain scan uses x.  The convolved sequence never goes to memory: one HBM round trip
// of x saved against a separate convolution kernel.
#include "scan_fwd.hpp"

extern "C" {

ssm_status ssm_conv_scan_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* dt,
                             const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                             const void* z, const float* h0, void* y, float* h_final, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return run_scan_fwd<true>(p, conv, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace, workspace_bytes,
                            stream);
}

ssm_status ssm_conv_state_update(const ssm_scan_params* p, const ssm_conv_params* conv, float* state, const void* x,
                                 const void* dt, const float* dt_bias, const float* A, const void* B, const void* C,
                                 const float* Dskip, const void* z, void* y, void* stream) {
  return run_state_update<true>(p, conv, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream);
}

}  // extern "C"
