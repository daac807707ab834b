// Host sanitizer build of the validation layer (test infrastructure): the
// kernel launchers and device-side helpers moe_api.cpp calls, replaced by
// stubs that enqueue nothing and report a launch failure, so that every path
// an argument check lets through ends at a launch error instead of a GPU.
#include "../../bit_dequant_expert_route_amd/csrc/moe_internal.h"

namespace moe_impl {

thread_local LaunchEvents g_launch_events;

hipError_t launch_head(const HeadParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_topk(const TopkParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gateup(const GateUpParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_down(const DownParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_partials(const PartialsParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_combine(const CombineParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fill(const FillParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_zero(void *, size_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_copy_f32(float *, const float *, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gdn_in(const GdnInParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gdn_step(const GdnParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_tier_reset(uint8_t *, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_tier_route(const TierRouteParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_route_group(const RouteGroupParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_router_tile(const void *, int, int, int, void *, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gateup_grouped(const GroupedParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_down_grouped(const GroupedParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_combine_tokens(const CombineTokensParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t noalloc_scratch(void **) { return hipErrorInvalidValue; }
// sizes: any positive value does for argument checks
size_t xstage_pair_bytes(int cols, int bits) { return (size_t)cols * 4 + (size_t)bits; }
size_t xstage_sum_bytes(int cols, int bits) { return (size_t)cols + (size_t)bits; }
bool combine_takes_partials(int, int, int, int) { return true; }

}  // namespace moe_impl
