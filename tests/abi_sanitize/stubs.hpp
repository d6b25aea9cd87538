// What the stand-in launchers of stubs.cpp record about the last launch.
#pragma once

#include "internal.hpp"

struct LaunchRecord {
  const char *fn = nullptr;
  int B = 0, T = 0, H = 0, KV = 0, D = 0, window = 0, T_max = 0, stages = 0;
  float scale = 0.f;
  void *workspace = nullptr;
  long count = 0;
};

extern LaunchRecord g_last;
void *fake_scratch();
