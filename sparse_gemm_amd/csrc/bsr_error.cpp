// bsr_error.cpp -- the per-thread error message behind bsr_last_error (host only, no HIP).
#include <string>

#include "bsr_internal.hpp"

namespace bsr {

namespace {
thread_local std::string g_last_error;
}  // namespace

int32_t fail(int32_t status, const std::string &msg) {
    g_last_error = msg;
    return status;
}

const char *last_error() { return g_last_error.c_str(); }

}  // namespace bsr
