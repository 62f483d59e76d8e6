// dg_host_stub.cpp -- host-only stand-ins for the device side of libdg.so, so that the
// C ABI's validation and planning (dg_api.cpp, compiled unchanged) can be built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run without a GPU.
//
//  * dg::kernel_configs: the library's own configuration rows (DG_CONFIG_TABLE), with
//    launchers that record the launch parameters instead of launching;
//  * the cast and sA-transform launchers: they count calls;
//  * the three HIP runtime queries the dispatcher makes: one device of 256 CUs.
#include "../../fp8_block_scaled_e4m3_amd/csrc/dg_internal.h"

namespace dg {

GemmParams g_last_params;
int g_last_grid = 0;
int g_last_config = -1;
int g_launches = 0;
int g_aux_launches = 0;

namespace {

template <int ID>
hipError_t record_launch(const GemmParams& p, int grid, hipStream_t) {
    g_last_params = p;
    g_last_grid = grid;
    g_last_config = ID;
    ++g_launches;
    return hipSuccess;
}

hipError_t one_per_cu(int* blocks) {
    *blocks = 1;
    return hipSuccess;
}

#define DG_STUB_CFG(ID, LAYOUT, BM, BN, WM, WN, WK, MF, NST, EFF, PIPE_OK, ALL_FMT, SPEC) \
    {ID, LAYOUT, BM, BN, WM, WN, WK, EFF, ALL_FMT, SPEC, &record_launch<ID>, &one_per_cu},

const KernelConfig kStubConfigs[] = {DG_CONFIG_TABLE(DG_STUB_CFG)};

}  // namespace

const KernelConfig* kernel_configs(int* count) {
    *count = (int)(sizeof(kStubConfigs) / sizeof(kStubConfigs[0]));
    return kStubConfigs;
}

hipError_t launch_quant_1x128(const void*, int, long, int, int, uint8_t*, long, float*, long, int, hipStream_t) {
    ++g_aux_launches;
    return hipSuccess;
}

hipError_t launch_quant_128x128(const void*, int, long, int, int, uint8_t*, long, float*, int, hipStream_t) {
    ++g_aux_launches;
    return hipSuccess;
}

hipError_t launch_sa_mn_major(const float*, long, float*, long, int, int, int, hipStream_t) {
    ++g_aux_launches;
    return hipSuccess;
}

}  // namespace dg

extern "C" {

hipError_t hipGetDevice(int* device) {
    *device = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
    *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

}  // extern "C"
