// Launcher stubs for the host-only sanitizer build of the C ABI.
//
// The host layer (vmla_api.cpp) is compiled with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer and linked against these stubs instead of the
// gfx950 kernels, so a call that passes validation reaches a stub, is counted,
// and returns hipErrorNoDevice (VMLA_ERR_HIP at the ABI) without touching any
// device. Fake pointers are therefore safe in that build. CPU tests only.
#include "kernels.h"

namespace {
int g_launches = 0;

hipError_t counted() {
  ++g_launches;
  return hipErrorNoDevice;
}
}  // namespace

namespace vmla {
hipError_t launch_append(const AppendArgs&, bool, hipStream_t) { return counted(); }
hipError_t launch_qprologue(const QArgs&, bool, hipStream_t) { return counted(); }
hipError_t launch_latent_attn(const AttnArgs&, bool, hipStream_t) { return counted(); }
hipError_t launch_latent_attn_wide(const AttnArgs&, hipStream_t) { return counted(); }
hipError_t launch_gemm(const GemmArgs&, int, int, hipStream_t) { return counted(); }
hipError_t launch_fold_query(const FoldArgs&, bool, hipStream_t) { return counted(); }
hipError_t launch_fold_output(const FoldArgs&, bool, hipStream_t) { return counted(); }
hipError_t launch_explicit_attn(const ExplicitArgs&, bool, hipStream_t) { return counted(); }
hipError_t launch_pack_kv(const FoldArgs&, bool, hipStream_t) { return counted(); }
hipError_t scratch_buffer(void**) { return hipErrorNoDevice; }
}  // namespace vmla

// Number of launcher calls reached so far (present only in the stub build).
extern "C" int vmla_stub_launch_count(void) { return g_launches; }
