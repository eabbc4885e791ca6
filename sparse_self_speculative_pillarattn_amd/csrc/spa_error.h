// spa_error.h -- the per-thread message behind spa_last_error (internal to libspa).
#pragma once
#include <stdint.h>

#include <string>

namespace spa {
// Records msg as this host thread's last error and returns code.
int32_t set_error(int32_t code, const std::string& msg);
}  // namespace spa
