// Internal declarations shared by the host and device translation units.
#pragma once
#include "../../include/kvpaged.h"

// Record a message for kv_last_error() and return `st`.
kv_status kvp_fail(kv_status st, const char* fmt, ...);
