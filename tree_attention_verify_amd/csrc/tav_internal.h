// Internal helpers of libtreeverify (host error reporting, launch checks,
// device bit helpers).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "treeverify.h"

namespace tav {

// Collects every failed argument check of one call, so the caller sees all
// blockers at once.
struct Checks {
    std::string msg;
    tav_status status = TAV_OK;
    // The first failed check decides the status; every message is kept.
    void fail(tav_status s, const std::string &what) {
        if (status == TAV_OK)
            status = s;
        if (!msg.empty())
            msg += "; ";
        msg += what;
    }
};

// TAV_NEED(checks, ok, status, message...): records the failure when `ok` is
// false.  The message is formed only then, so a call whose arguments pass
// builds no strings (host time per call matters for small launches).
#define TAV_NEED(chk, ok, st, ...)            \
    do {                                      \
        if (!(ok))                            \
            (chk).fail((st), __VA_ARGS__);    \
    } while (0)

void set_error(const char *fn, const std::string &msg);
void clear_error();
tav_status finish(const char *fn, Checks &c);          // records c, returns its status
tav_status launched(const char *fn);                   // checks hipGetLastError()

inline std::string str(long long v) { return std::to_string(v); }

inline bool is_pow2(long long v) { return v > 0 && (v & (v - 1)) == 0; }

inline int ilog2(long long v) {
    int s = 0;
    while ((1LL << s) < v)
        ++s;
    return s;
}

}  // namespace tav
