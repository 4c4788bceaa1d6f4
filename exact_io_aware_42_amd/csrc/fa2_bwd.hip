#include "fa2_launch.hpp"
namespace fa2 {
hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }
}
