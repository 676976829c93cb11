// Thread-local error text behind nomas_last_error(), shared by the files that
// implement C ABI entry points.
#pragma once

#include <string>

#include "nomas_attn.h"

namespace nomas {

nomas_status set_error(nomas_status s, const std::string& what);  // records `what`, returns s
nomas_status clear_error();                                       // returns NOMAS_OK

}  // namespace nomas
