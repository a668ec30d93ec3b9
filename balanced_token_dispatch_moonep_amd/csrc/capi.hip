// Host-only parts of the C ABI: error strings and version.
#include "common.h"

extern "C" const char* moonep_strerror(int code) {
    switch (code) {
        case MOONEP_OK: return "ok";
        case MOONEP_EINVAL: return "invalid argument (dims or NULL pointer)";
        case MOONEP_EALIGN: return "pointer not 16-byte aligned";
        case MOONEP_EHIP: return "HIP launch failed";
        case MOONEP_ENOTSUP: return "unsupported combination of dims/flags";
        case MOONEP_ETOOBIG: return "plan workspace larger than the static workspace of moonep_plan_noalloc";
        default: return "unknown error";
    }
}

extern "C" const char* moonep_version(void) { return "moonep-mi355x 0.1 (gfx950)"; }
