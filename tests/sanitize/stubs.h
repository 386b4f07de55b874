// Call log of the host-only kernel launchers (kernel_stubs.cpp).
#pragma once
namespace kq {
struct StubLog {
  long stage, gemv, fill, read, tile, probe, gather, softmax;
  unsigned device_word;  // what read_device_word reports
  char violation[160];   // first launch-description invariant that failed
};
extern StubLog g_stub;
}  // namespace kq
