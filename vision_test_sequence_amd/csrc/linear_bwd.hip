#include "common.hpp"
#include "internal.hpp"
namespace ttt {
size_t lin_bwd_ws_bytes(int, int, int) { return 0; }
hipError_t launch_lin_bwd(LinBwdLaunch, hipStream_t) { return hipErrorNotSupported; }
}
