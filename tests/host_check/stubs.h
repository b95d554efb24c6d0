// What the stand-in launchers of stubs.cpp recorded.
#pragma once

struct HostCheckLog {
  int calls = 0;
  const char* last = "";
  int n = 0, n_kv = 0, q_start = 0, head_dim = 0, split = 0;
  bool fail_launch = false;  // make the next launches report a HIP error
};
extern HostCheckLog g_log;
