// Test-only stand-ins for the kernel launchers, so that the C-ABI host code can be
// built for the host alone with sanitizers (the host checks never reach a launch:
// every stub reports itself and fails if one is called).
#include <cstdio>

#include "common.hpp"

namespace vdit {

static hipError_t stub(const char* name) {
  std::printf("FAIL: launcher %s reached on a validation path\n", name);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd(const AttnArgs&, int, bool, bool, hipStream_t) { return stub("attn_fwd"); }
hipError_t launch_attn_sparse(const AttnArgs&, int, hipStream_t) { return stub("attn_sparse"); }
hipError_t launch_vsa_means(const VsaMeanArgs&, int, hipStream_t) { return stub("vsa_means"); }
hipError_t launch_vsa_select(const VsaSelectArgs&, hipStream_t) { return stub("vsa_select"); }
hipError_t launch_prepare(const PrepArgs&, int, bool, hipStream_t) { return stub("prepare"); }
hipError_t launch_quantize(const QuantArgs&, int, hipStream_t) { return stub("quantize"); }
hipError_t launch_pack(const void*, void*, int64_t, int32_t, int32_t, int32_t, bool, hipStream_t) {
  return stub("pack");
}
hipError_t launch_rope_probe(const RopeGeom&, int32_t, int32_t, int32_t*, hipStream_t) { return stub("rope_probe"); }

}  // namespace vdit
