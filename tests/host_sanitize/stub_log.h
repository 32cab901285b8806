// What the stand-in launchers of hip_stubs.cpp record.
#pragma once
#include <hip/hip_runtime.h>

struct StubLog {
    int device = 0;                                // the current device ordinal
    const char *arch = "gfx950:sramecc+:xnack-";   // that device's architecture name
    hipError_t result = hipSuccess;               // what every launcher returns
    int calls = 0;                                 // launcher calls so far
    char last[64] = "";                            // the last launcher called
    long long a = 0, b = 0, c = 0;                 // its leading size arguments
};
extern StubLog g_stub;
