// Launch records of the host stand-ins (see stub_launchers.cpp).
#pragma once
#include "dsa_kernels.hpp"

namespace stub {
struct Launch {
  const char* what = nullptr;
  int n = 0, n_seq = 0, page_size = 0;
  dsa::MqaArgs mqa{};
  const uint16_t* p_ws = nullptr;
  const uint16_t* ds_ws = nullptr;
};
extern Launch last;
extern int launches;
extern unsigned char scratch_stand_in[64];
}  // namespace stub
