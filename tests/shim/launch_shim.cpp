// Test-only stand-in for hipLaunchKernel (preloaded into a subprocess on a
// machine without a GPU): every launch of a real schedule is recorded, not
// run. For each GEMM with split-K partials and each key-split attention it
// checks that the partials it would write end before the tile counters,
// which the workspace places right after the partial buffer; a violation is
// reported on stderr as "OVERFLOW ...". At exit it prints the launch count.
#include <hip/hip_runtime.h>
#include <cctype>
#include <dlfcn.h>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>
#include "gemm.h"
#include "attention.h"

namespace {
long g_launches = 0;
uintptr_t g_cnt = 0;   // tile counters of the current workspace (from the GEMMs)
struct Pending { uintptr_t end; std::string what; };
std::vector<Pending> g_attn;   // key-split attention partial ends, checked once g_cnt is known

// integer template arguments of a mangled kernel name, in order (each is
// encoded as L<type><value>E, e.g. Li96E)
std::vector<long> iargs(const char* m) {
  std::vector<long> out;
  for (const char* p = m; *p; p++) {
    if (p[0] == 'L' && p[1] == 'i' && (isdigit((unsigned char)p[2]) || p[2] == 'n')) {
      const char* q = p + 2;
      const bool neg = *q == 'n';
      if (neg) q++;
      long v = 0;
      while (isdigit((unsigned char)*q)) v = v * 10 + (*q++ - '0');
      if (*q == 'E') out.push_back(neg ? -v : v);
    }
  }
  return out;
}
struct Report {
  ~Report() {
    for (const auto& p : g_attn)
      if (g_cnt && p.end > g_cnt) fprintf(stderr, "OVERFLOW %s\n", p.what.c_str());
    fprintf(stderr, "launches %ld\n", g_launches);
  }
} g_report;
}  // namespace

extern "C" hipError_t hipLaunchKernel(const void* fn, dim3 grid, dim3, void** args, size_t, hipStream_t) {
  g_launches++;
  Dl_info di{};
  if (!dladdr(fn, &di) || !di.dli_sname) return hipSuccess;
  const std::string name = di.dli_sname;
  const std::vector<long> t = iargs(di.dli_sname);
  if (name.find("k_gemm") != std::string::npos && t.size() >= 4) {
    // k_gemm<WT, CT, MB, WN, WK, NBW, ...>: integers MB, WN, WK, NBW first
    vla::GemmArgs a;
    memcpy(&a, args[0], sizeof(a));
    const long BM = 16 * t[0], BN = 16 * t[3] * t[1];
    g_cnt = (uintptr_t)a.cnt_tile;
    if (a.split > 1) {
      const uintptr_t end = (uintptr_t)a.part + (uintptr_t)a.split * a.n_tiles_m * a.n_tiles_n * BM * BN * 4;
      if (end > (uintptr_t)a.cnt_tile)
        fprintf(stderr, "OVERFLOW gemm M %d N %d K %d split %d tiles %dx%d: partials end %zu bytes past the counters\n", a.M,
                a.N, a.K, a.split, a.n_tiles_m, a.n_tiles_n, (size_t)(end - (uintptr_t)a.cnt_tile));
    }
  } else if (name.find("k_attention") != std::string::npos && t.size() >= 2) {
    vla::AttnArgs a;
    memcpy(&a, args[0], sizeof(a));
    if (a.nsplit > 1) {
      const long dp = t[0];   // k_attention<CT, DP, HPW>
      const uintptr_t end = (uintptr_t)a.part + (uintptr_t)grid.x * 4 * 16 * (dp + 2) * 4;
      char buf[160];
      snprintf(buf, sizeof(buf), "attention Sq %d Sk %d nsplit %d: partials past the counters", a.Sq, a.Sk, a.nsplit);
      g_attn.push_back({end, buf});
    }
  }
  return hipSuccess;
}
extern "C" hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) { return hipSuccess; }
