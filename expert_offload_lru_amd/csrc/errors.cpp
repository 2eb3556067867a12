#include "errors.hpp"

#include "moe_offload.h"

namespace moe {
namespace {
thread_local std::string g_last_error;
}
int set_error(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}
}  // namespace moe

extern "C" const char *moe_last_error(void) { return moe::g_last_error.c_str(); }
