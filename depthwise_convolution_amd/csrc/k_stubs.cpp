// k_stubs.cpp -- planners of kernel families not built into this library yet.
#include "plan.h"

namespace dw {

bool plan_ldstile(Plan &) { return false; }

}  // namespace dw
