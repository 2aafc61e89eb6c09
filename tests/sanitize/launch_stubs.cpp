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
hipError_t launch_bwd_reverse(int, const BwdArgs&, void*, void*, void*, float*, hipStream_t) { STUB; }
hipError_t launch_bwd_scale_rev(int, const BwdArgs&, int, void*, hipStream_t) { STUB; }
hipError_t launch_bwd_onehot(int64_t, int, int, float*, hipStream_t) { STUB; }
hipError_t launch_bwd_sum_rev(int, const BwdArgs&, const void*, int64_t, int, float*, hipStream_t) { STUB; }
hipError_t launch_bwd_rowdot(int, const BwdArgs&, const void*, int, hipStream_t) { STUB; }
hipError_t launch_bwd_gate(int, const BwdArgs&, const float*, float*, hipStream_t) { STUB; }
hipError_t launch_ccq_fill(int64_t, int, float*, float*, hipStream_t) { STUB; }
hipError_t launch_ccq_ksum(int, int, int, int, int, int, const void*, float*, hipStream_t) { STUB; }
hipError_t launch_ccq_combine(int, int, int, int, int, int, const void*, const void*, const void*, const float*,
                              const float*, const float*, void*, hipStream_t) { STUB; }
hipError_t launch_decode_step(int, int, const DecodeArgs&, hipStream_t) { STUB; }
hipError_t launch_gdn_wy(int, int, int, const GdnArgs&, hipStream_t) { STUB; }
hipError_t launch_gdn_state(int, int, int, const GdnArgs&, hipStream_t) { STUB; }
hipError_t launch_lambda_mlp(int64_t, int, int, const float*, const float*, const float*, const float*, float*,
                             hipStream_t) { STUB; }
}  // namespace llattn
