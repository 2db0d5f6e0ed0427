// Launch unit of the head_dim-512 paged prefill kernel, compiled on its own so
// that its MFMA accumulators take the accumulator-register form (O fills the
// 256 accumulator registers; the scores use inline-assembly MFMAs with VGPR
// accumulators).
#include "psw_prefill512.hpp"

namespace psw_dev {

hipError_t launch_prefill512(bool out_bf16, const AttnParams& p, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const dim3 grid(n_items * p.num_kv_heads);
  const bool p16 = p.ps.page_size == 16;
  if (out_bf16) {
    if (p16) hipLaunchKernelGGL((prefill512_kernel<true, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prefill512_kernel<true, false>), grid, dim3(256), 0, s, p);
  } else {
    if (p16) hipLaunchKernelGGL((prefill512_kernel<false, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prefill512_kernel<false, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace psw_dev
