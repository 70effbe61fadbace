// Stand-alone driver of the C++ oracle: reads one problem and its inputs from
// a directory of raw files, runs ox_run and writes the outputs back as raw
// files.  TEST INFRASTRUCTURE ONLY: the tests build it (with the address and
// undefined-behaviour sanitizers) to run the oracle outside Python.
//
//   run_case DIR
//
// DIR/problem.txt holds "key value" lines: num_groups valid_m n k ab act d_fp8
// c_out srelu_s glu_gamma geglu_alpha linear_offset clamp_min clamp_max
// norm_const nrows.  Inputs (absent file = NULL pointer): a.bin sfa.bin b.bin
// sfb.bin po.bin alpha.bin beta.bin prob.bin c_in.bin rows.bin (int64).
// Outputs: group.bin cr.bin d.bin dprob.bin c_bits.bin d_bits.bin d_code.bin
// sfd_row.bin d_col_code.bin sfd_col.bin amax.bin, each sized by the caller's
// expectation of the problem (see oracle.h).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <iterator>
#include <map>
#include <string>
#include <vector>

#include "oracle.h"

namespace {

std::vector<char> slurp(const std::string& path, bool* found) {
  std::ifstream f(path, std::ios::binary);
  *found = static_cast<bool>(f);
  if (!f) return {};
  return std::vector<char>(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
}

void spill(const std::string& path, const void* p, size_t bytes) {
  std::ofstream f(path, std::ios::binary);
  f.write(static_cast<const char*>(p), static_cast<std::streamsize>(bytes));
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: run_case DIR\n");
    return 2;
  }
  const std::string dir = argv[1];
  std::map<std::string, double> kv;
  {
    // values through strtod, which also reads "inf" and "-inf"
    std::ifstream f(dir + "/problem.txt");
    std::string key, val;
    while (f >> key >> val) kv[key] = std::strtod(val.c_str(), nullptr);
  }
  for (const char* key : {"num_groups", "valid_m", "n", "k", "ab", "act", "d_fp8", "c_out", "srelu_s", "glu_gamma",
                          "geglu_alpha", "linear_offset", "clamp_min", "clamp_max", "norm_const", "nrows"})
    if (!kv.count(key)) {
      std::fprintf(stderr, "problem.txt lacks %s\n", key);
      return 2;
    }
  ox_problem p{};
  p.num_groups = static_cast<int32_t>(kv["num_groups"]);
  p.valid_m = static_cast<int64_t>(kv["valid_m"]);
  p.n = static_cast<int32_t>(kv["n"]);
  p.k = static_cast<int32_t>(kv["k"]);
  p.ab = static_cast<int32_t>(kv["ab"]);
  p.act = static_cast<int32_t>(kv["act"]);
  p.d_fp8 = static_cast<int32_t>(kv["d_fp8"]);
  p.c_out = static_cast<int32_t>(kv["c_out"]);
  p.srelu_s = kv["srelu_s"];
  p.glu_gamma = kv["glu_gamma"];
  p.geglu_alpha = kv["geglu_alpha"];
  p.linear_offset = kv["linear_offset"];
  p.clamp_min = kv["clamp_min"];
  p.clamp_max = kv["clamp_max"];
  p.norm_const = static_cast<float>(kv["norm_const"]);
  const int64_t nrows = static_cast<int64_t>(kv["nrows"]);

  std::map<std::string, std::vector<char>> in;
  std::map<std::string, bool> have;
  for (const char* name : {"a", "sfa", "b", "sfb", "po", "alpha", "beta", "prob", "c_in", "rows"}) {
    bool found = false;
    in[name] = slurp(dir + "/" + name + ".bin", &found);
    have[name] = found;
  }
  auto ptr = [&](const char* name) -> const void* { return have[name] ? in[name].data() : nullptr; };
  ox_inputs inputs{};
  inputs.a = ptr("a");
  inputs.sfa = static_cast<const uint8_t*>(ptr("sfa"));
  inputs.b = ptr("b");
  inputs.sfb = static_cast<const uint8_t*>(ptr("sfb"));
  inputs.padded_offsets = static_cast<const int32_t*>(ptr("po"));
  inputs.alpha = static_cast<const float*>(ptr("alpha"));
  inputs.beta = static_cast<const float*>(ptr("beta"));
  inputs.prob = static_cast<const float*>(ptr("prob"));
  inputs.c_in = static_cast<const uint16_t*>(ptr("c_in"));
  const int64_t* rows = static_cast<const int64_t*>(ptr("rows"));

  const int64_t n = p.n;
  const int64_t no = (p.act == OX_SWIGLU || p.act == OX_GEGLU) ? n / 2
                     : (p.act == OX_DSWIGLU || p.act == OX_DGEGLU) ? 2 * n : n;
  const bool pairs_amax = (p.act == OX_DSWIGLU || p.act == OX_DGEGLU) && p.ab != OX_BF16 && !p.d_fp8;
  std::vector<int32_t> group(nrows);
  std::vector<double> cr(nrows * n), d(nrows * no), dprob(nrows), amax(p.num_groups * (pairs_amax ? 2 : 1));
  std::vector<uint16_t> c_bits(nrows * n), d_bits(nrows * no);
  std::vector<uint8_t> d_code(nrows * no), sfd_row(nrows * (no / 32)), d_col_code(nrows * no),
      sfd_col(no * (nrows / 32 > 0 ? nrows / 32 : 1));
  ox_outputs out{group.data(), cr.data(), d.data(), dprob.data(), c_bits.data(), d_bits.data(), d_code.data(),
                 sfd_row.data(), d_col_code.data(), sfd_col.data(), amax.data()};
  if (ox_run(&p, &inputs, rows, nrows, &out)) {
    std::fprintf(stderr, "ox_run: %s\n", ox_last_error());
    return 1;
  }
  spill(dir + "/group.out", group.data(), group.size() * sizeof(int32_t));
  spill(dir + "/cr.out", cr.data(), cr.size() * sizeof(double));
  spill(dir + "/d.out", d.data(), d.size() * sizeof(double));
  spill(dir + "/dprob.out", dprob.data(), dprob.size() * sizeof(double));
  spill(dir + "/c_bits.out", c_bits.data(), c_bits.size() * sizeof(uint16_t));
  spill(dir + "/d_bits.out", d_bits.data(), d_bits.size() * sizeof(uint16_t));
  spill(dir + "/d_code.out", d_code.data(), d_code.size());
  spill(dir + "/sfd_row.out", sfd_row.data(), sfd_row.size());
  spill(dir + "/d_col_code.out", d_col_code.data(), d_col_code.size());
  spill(dir + "/sfd_col.out", sfd_col.data(), sfd_col.size());
  spill(dir + "/amax.out", amax.data(), amax.size() * sizeof(double));
  return 0;
}
