// Status strings of the DLRM sparse C ABI.
#include "dlrm_sparse.h"

extern "C" const char *dlrm_status_string(int status) {
    switch (status) {
        case DLRM_OK: return "ok";
        case DLRM_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or misalignment)";
        case DLRM_ERR_UNSUPPORTED: return "unsupported shape or size for this library";
        case DLRM_ERR_HIP: return "HIP launch or runtime call failed";
        case DLRM_ERR_INDEX_RANGE: return "offsets or indices out of range (device check)";
        case DLRM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown status";
    }
}
