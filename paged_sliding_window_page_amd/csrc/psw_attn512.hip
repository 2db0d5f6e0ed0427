// Instantiations of the paged attention kernel for head_dim 512 in its split-KV
// form (one-token decode with a GQA group wider than the decode kernel's).
// Each head_dim is its own translation unit so that it can be compiled with
// the code-generation options that suit its register budget.
#include "psw_attention.hpp"

namespace psw_dev {
namespace {

template <bool SPLIT, bool OB>
hipError_t launch_one(const AttnParams& p, int n_items, hipStream_t s) {
  const dim3 grid(n_items * p.num_kv_heads);
  if (p.ps.page_size == 16)
    hipLaunchKernelGGL((attention_kernel<512, SPLIT, OB, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attention_kernel<512, SPLIT, OB, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_d512(bool split, bool out_bf16, const AttnParams& p, int n_items,
                                hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  // prefill: its own kernel (psw_prefill512.hip); here the split-KV form
  if (!split) return launch_prefill512(out_bf16, p, n_items, s);
  return out_bf16 ? launch_one<true, true>(p, n_items, s) : launch_one<true, false>(p, n_items, s);
}

hipError_t launch_merge_d512(bool out_bf16, MergeParams p, const int32_t* req_splits,
                             const int32_t* qo_indptr, int batch, hipStream_t s) {
  for (int b0 = 0; b0 < batch; b0 += kMergeReqsPerLaunch) {
    const int n = batch - b0 < kMergeReqsPerLaunch ? batch - b0 : kMergeReqsPerLaunch;
    bool any = false;
    for (int i = 0; i < n; ++i) {
      p.req[3 * i] = req_splits[2 * (b0 + i)];
      p.req[3 * i + 1] = req_splits[2 * (b0 + i) + 1];
      p.req[3 * i + 2] = qo_indptr[b0 + i];
      any = any || p.req[3 * i + 1] > 0;
    }
    if (!any) continue;
    const dim3 grid(p.num_qo_heads, n);
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<512, true>), grid, dim3(512 / 4), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<512, false>), grid, dim3(512 / 4), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace psw_dev
