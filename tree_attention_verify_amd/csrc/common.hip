// Error reporting of libtreeverify.
#include "tav_internal.h"

namespace tav {

static thread_local std::string g_last_error;

void set_error(const char *fn, const std::string &msg) {
    g_last_error = std::string(fn) + ": " + msg;
}

void clear_error() { g_last_error.clear(); }

tav_status finish(const char *fn, Checks &c) {
    if (c.status == TAV_OK)
        clear_error();
    else
        set_error(fn, c.msg);
    return c.status;
}

tav_status launched(const char *fn) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error(fn, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return TAV_ERR_HIP;
    }
    clear_error();
    return TAV_OK;
}

}  // namespace tav

extern "C" const char *tav_last_error(void) { return tav::g_last_error.c_str(); }

extern "C" const char *tav_version(void) { return "treeverify 0.1 gfx950"; }
