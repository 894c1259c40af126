/* The status string of any int, called the way a C caller may: in C an
 * enum-typed argument may carry any int value. */
#include "rglru.h"

const char* host_abi_status_of_int(int v) { return rglru_status_string((rglru_status_t)v); }
