#include "fa_common.hpp"
#include "fa_internal.h"
namespace fa {
hipError_t launch_bwd(BwdArgs, int, bool, hipStream_t) { return hipErrorNotSupported; }
}
