// Stand-ins for the kernel launchers of libllattn (declared in
// fenwick_tree_linear_amd/csrc/ll_launch.hpp), so that the C ABI's host code
// (api.cpp: validation, workspace planning, launch sequencing, kernel timing)
// can be built with host sanitizers and driven without a GPU.  Every stub
// reports a failed launch.  Test infrastructure only.
#include "ll_launch.hpp"

namespace llattn {
#define STUB return hipErrorInvalidValue
hipError_t launch_block_state(int, int, int, const PrefillArgs&, hipStream_t) { STUB; }
hipError_t launch_chunk_attn(int, int, int, const PrefillArgs&, hipStream_t) { STUB; }
hipError_t launch_fenwick_scan(int, const PrefillArgs&, hipStream_t) { STUB; }
hipError_t launch_state_export(int, int, const PrefillArgs&, hipStream_t) { STUB; }
hipError_t launch_prior_read(int, int, int, const PrefillArgs&, hipStream_t) { STUB; }
hipError_t launch_bwd_native(int, int, int, const BwdArgs&, const BwdFwdNodes&, const BwdWork&, int, hipStream_t) {
  STUB;
}
hipError_t launch_ccq_prepare(int, int, int, int, int, int, const void*, float*, int64_t, int, float*, float*,
                              hipStream_t) { STUB; }
hipError_t launch_ccq_combine(int, int, int, int, int, int, const void*, const void*, const void*, const float*,
                              const float*, const float*, void*, hipStream_t) { STUB; }
hipError_t launch_decode_step(int, int, int, const DecodeArgs&, hipStream_t) { STUB; }
hipError_t launch_pad_copy(int, const void*, void*, int64_t, int, int, int, int, int, int, hipStream_t) { STUB; }
hipError_t launch_gdn_wy(int, int, int, const GdnArgs&, hipStream_t) { STUB; }
hipError_t launch_gdn_state(int, int, int, const GdnArgs&, hipStream_t) { STUB; }
hipError_t launch_lambda_mlp(int64_t, int, int, const float*, const float*, const float*, const float*, float*,
                             hipStream_t) { STUB; }
}  // namespace llattn
