// Thread-local error message of the C ABI.
#pragma once
#include <string>

namespace moe {
int set_error(int code, const std::string &msg);   // returns code
}
