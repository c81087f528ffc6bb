// host_common.cpp -- status strings, thread-local error detail and the device check.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.hpp"

namespace lsa {

static thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_err[0] = '\0'; }

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
int g_dev_cus[kMaxDevices];
}  // namespace

int check_device(int* num_cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LSA_ERR_UNSUPPORTED, "device id %d", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(LSA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        g_dev_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        g_dev_cus[dev] = prop.multiProcessorCount;
    }
    if (g_dev_state[dev] != 1)
        return fail(LSA_ERR_UNSUPPORTED, "this library is built for gfx950 (MI355X) only");
    if (num_cus) *num_cus = g_dev_cus[dev];
    return LSA_OK;
}

int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LSA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return LSA_OK;
}

}  // namespace lsa

extern "C" const char* lsa_status_string(int status) {
    switch (status) {
        case LSA_OK: return "ok";
        case LSA_ERR_INVALID_ARG: return "invalid argument";
        case LSA_ERR_UNSUPPORTED: return "unsupported shape or device";
        case LSA_ERR_WORKSPACE: return "workspace too small";
        case LSA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* lsa_last_error(void) { return lsa::g_err; }

extern "C" int lsa_version(void) { return 100; }

size_t lsa_select_workspace(int B, int64_t max_len);
size_t lsa_topk_workspace(int B, int64_t max_len);
size_t lsa_attend_workspace(int dtype, int B, int T, int Hq, int Dl, int k, int64_t max_hca);

extern "C" size_t lsa_workspace_bytes(int op, int B, int T, int Hq, int Dl, int64_t max_len,
                                      int k, int64_t max_hca) {
    if (B <= 0) return 0;
    switch (op) {
        case LSA_OP_SELECT: return max_len < 0 ? 0 : lsa_select_workspace(B, max_len);
        case LSA_OP_TOPK: return max_len < 0 ? 0 : lsa_topk_workspace(B, max_len);
        case LSA_OP_ATTEND:
            // sized for the bf16 matrix-core path (the fp32 path needs none)
            if (T <= 0 || Hq <= 0 || Dl <= 0 || k <= 0) return 0;
            return lsa_attend_workspace(LSA_DTYPE_BF16, B, T, Hq, Dl, k,
                                        max_hca > 0 ? max_hca : 0);
        default: return 0;
    }
}
