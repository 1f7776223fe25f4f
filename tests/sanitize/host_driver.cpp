// Driver for the sanitized host build of libstc (tests/test_host_sanitized.py).
// Reads one command per line on stdin and prints the library's answer on one
// line of stdout, so the test can compare it with the oracle:
//   ds b                       -> stc_delta_star(b)
//   tb avg d                   -> stc_total_bits(avg, d)
//   wf d B l_0 .. l_{d-1}      -> status bits_0 .. bits_{d-1}
//   al d B variant param l_0.. -> status bits_0 .. (stc_allocate_bits)
//   eh d a_00 a_01 ..          -> status lambda_0 .. U_00 U_01 .. (stc_eigh)
//   lm n levels tol iters s_0..-> status iters c_0 .. (stc_lloyd_max)
//   inv                        -> statuses of calls with invalid arguments
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/stc.h"

static void invalid_calls() {
  std::vector<int> st;
  stc_head_info info{};
  std::vector<unsigned char> blob(64);
  // NULL or misaligned buffers, bad sizes: rejected before any device work
  st.push_back(stc_encode_kv(&info, nullptr, 10, nullptr, STC_BF16, 128, nullptr, nullptr, nullptr));
  st.push_back(stc_decode_kv(nullptr, nullptr, 10, nullptr, nullptr, nullptr, STC_BF16, 128, nullptr));
  st.push_back(stc_encode_kv_batched(nullptr, 0, nullptr, nullptr, 1, 10, nullptr, STC_BF16, 128, 1280, nullptr, 16,
                                     nullptr, nullptr));
  st.push_back(stc_attend_compressed_batched(nullptr, 1, nullptr, nullptr, &info, 1, 10, nullptr, nullptr, 16, 4,
                                             nullptr, nullptr, 0.1f, nullptr, 0, nullptr));
  st.push_back(stc_calibrate_head(64, 10, nullptr, STC_BF16, 64, 2.0f, nullptr, STC_XFORM_EIGEN, &info, nullptr,
                                  nullptr));
  st.push_back(stc_calibrate_head(128, 10, blob.data(), 7, 128, 2.0f, nullptr, STC_XFORM_EIGEN, &info, nullptr,
                                  nullptr));
  st.push_back(stc_check_state_map(nullptr, 3, 4, nullptr));
  st.push_back(stc_check_state_map(nullptr, -1, 4, nullptr));
  uint8_t bits[128];
  double lam[128];
  for (int j = 0; j < 128; ++j) lam[j] = 1.0 / (j + 1);
  st.push_back(stc_water_fill(128, lam, 8 * 128 + 1, bits));
  st.push_back(stc_water_fill(128, lam, -1, bits));
  st.push_back(stc_allocate_bits(128, lam, 256, 99, 0.0, bits));
  st.push_back(stc_allocate_bits(128, lam, 256, STC_ALLOC_GROUPED, 3.0, bits));
  double u[4], l2[2];
  const double nanm[4] = {1.0, 0.0, 0.0, __builtin_nan("")};
  st.push_back(stc_eigh(2, nanm, u, l2));
  st.push_back(stc_eigh(0, nanm, u, l2));
  for (size_t i = 0; i < st.size(); ++i) std::printf("%s%d", i ? " " : "", st[i]);
  std::printf("\n");
  // the messages are NUL-terminated strings
  std::printf("%zu\n", std::string(stc_last_error()).size() > 0 ? (size_t)1 : (size_t)0);
}

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    if (cmd == "ds") {
      int b;
      in >> b;
      std::printf("%.17g\n", stc_delta_star(b));
    } else if (cmd == "tb") {
      float avg;
      int d;
      in >> avg >> d;
      std::printf("%d\n", stc_total_bits(avg, d));
    } else if (cmd == "wf" || cmd == "al") {
      int d, B, variant = 0;
      double param = 0.0;
      in >> d >> B;
      if (cmd == "al") in >> variant >> param;
      std::vector<double> lam(d);
      for (auto& v : lam) in >> v;
      std::vector<uint8_t> bits(d, 0xEE);
      const int s = cmd == "wf" ? stc_water_fill(d, lam.data(), B, bits.data())
                                : stc_allocate_bits(d, lam.data(), B, variant, param, bits.data());
      std::printf("%d", s);
      for (auto b : bits) std::printf(" %d", b);
      std::printf("\n");
    } else if (cmd == "eh") {
      int d;
      in >> d;
      std::vector<double> a((size_t)d * d), u((size_t)d * d), lam(d);
      for (auto& v : a) in >> v;
      const int s = stc_eigh(d, a.data(), u.data(), lam.data());
      std::printf("%d", s);
      for (auto v : lam) std::printf(" %.17g", v);
      for (auto v : u) std::printf(" %.17g", v);
      std::printf("\n");
    } else if (cmd == "lm") {
      long long n;
      int levels, max_iter;
      double tol;
      in >> n >> levels >> tol >> max_iter;
      std::vector<double> smp((size_t)n), c(levels);
      for (auto& v : smp) in >> v;
      int iters = -1;
      const int s = stc_lloyd_max(smp.data(), n, levels, tol, max_iter, c.data(), &iters);
      std::printf("%d %d", s, iters);
      for (auto v : c) std::printf(" %.17g", v);
      std::printf("\n");
    } else if (cmd == "inv") {
      invalid_calls();
    }
    std::fflush(stdout);
  }
  return 0;
}
