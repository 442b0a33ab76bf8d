// Library identification and status texts.
#include "common.hpp"

extern "C" int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

extern "C" const char* fp8q_status_string(fp8q_status_t status) {
    switch (status) {
        case FP8Q_OK: return "ok";
        case FP8Q_ERR_INVALID_ARG: return "invalid argument";
        case FP8Q_ERR_UNSUPPORTED: return "unsupported shape, layout or alignment";
        case FP8Q_ERR_WORKSPACE: return "workspace too small";
        case FP8Q_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

extern "C" int fp8_abi_version(void) { return fp8q_abi_version(); }

extern "C" const char* fp8_status_string(fp8q_status_t status) { return fp8q_status_string(status); }
