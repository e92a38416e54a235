// Stand-ins for the kernel launchers, so that the C-ABI layer's host code
// (argument checks, workspace layout, launch-argument packing) can be built
// with g++ under the sanitizers and driven without a GPU.  Each stub records
// the call and reports success.  Test infrastructure only.
#include "../../vector_quantized_bit_vqkv_amd/csrc/internal.h"

int g_launches = 0;

// The C-ABI layer asks the runtime for error text and, for the split count it
// suggests, the current device's compute units (none here: it falls back).
const char* hipGetErrorString(hipError_t) { return "stubbed HIP runtime"; }
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }

namespace vqkv {
hipError_t launch_transform_query(const TransformQueryArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_append(const AppendArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_combine(const CombineArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_value_output_transform(const ValueOutputArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_smooth_scales(int, int, const void*, int, float*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_train_codebook(const TrainArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
// The static scratch's address: an aligned dummy (nothing dereferences it).
hipError_t static_scratch(void** addr, int* device) {
    *addr = reinterpret_cast<void*>(0x20000);
    if (device) *device = 0;
    return hipSuccess;
}
}  // namespace vqkv
