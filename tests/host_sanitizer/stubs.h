// Launch records of the host-only launcher stand-ins (stubs.cpp).
#pragma once
#include <cstdint>
#include <vector>

struct LaunchRecord {
    const char* what;   // launcher name
    int64_t rows;       // rows (or m) handed to it
    const void* in;     // principal input pointer
    const void* out;    // principal output pointer
    const void* aux;    // scales / weight codes / workspace
    const void* aux2;   // weight scales / activations (W4A4)
};

extern std::vector<LaunchRecord> g_launches;
extern bool g_fail_next;
