// fa_host_stubs.cpp -- stand-ins for the kernel launchers, for the host-only
// build of the C ABI that runs under the address and undefined-behaviour
// sanitizers (build.build_host_sanitized).  That build exists to check the
// host logic of fa_api.cpp (argument checks, workspace sizes, status codes);
// it has no device code, so every launcher here reports an error and computes
// nothing.  libfa.so never links this file.
#include "fa_kernels.hpp"

namespace fa {

hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_splitkv(const SplitArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_rowdot(float**) { return hipErrorNotSupported; }

}  // namespace fa
