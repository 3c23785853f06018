// Internal helpers shared by the library's host translation units.
#pragma once

#include <string>

namespace pkv {

void set_error(const std::string& msg);
void clear_error();

inline int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

}  // namespace pkv
