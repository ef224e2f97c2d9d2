#include "common.h"
#include "kernels.h"
namespace attn {
hipError_t launch_mla(const MlaParams&, bool, hipStream_t) { return hipErrorNotSupported; }
}
