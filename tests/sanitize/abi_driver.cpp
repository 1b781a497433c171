// Host-only driver of libhsq's C ABI for AddressSanitizer / UndefinedBehavior-
// Sanitizer builds of the library's host translation units (api.cpp, host.cpp).
// Nothing here touches a GPU: every call either runs host code only (the
// codebook, the tier plan, the workspace size) or fails argument validation
// before any launch.
//
// Commands, one per line on stdin:
//   codebook D BITS              -> "codebook RC c0 .. c(L-1) | t0 .. t(L-2)"
//   tier T NS NR GN NM m0 ..     -> "tier RC N1 NG | l1 .. | g .."
//   workspace B HQ HKV D N1 NG BETA GN -> "workspace BYTES"
//   errors                       -> "errors CHECKED" (mismatches on stderr)
// Output buffers are sized exactly (the tier plan's from a first call that
// only counts), so a write past the end is a sanitizer report.  Exit status 1
// when an argument check returned another code than the one the C ABI states.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "hsq.h"

namespace {

int g_checked = 0, g_bad = 0;

void expect(const char* what, long got, long want, const char* msg_part = nullptr) {
  ++g_checked;
  if (got != want) {
    std::fprintf(stderr, "MISMATCH %s: returned %ld, expected %ld (%s)\n", what, got, want,
                 hsq_last_error());
    ++g_bad;
    return;
  }
  if (msg_part && !std::strstr(hsq_last_error(), msg_part)) {
    std::fprintf(stderr, "MISMATCH %s: message '%s' lacks '%s'\n", what, hsq_last_error(),
                 msg_part);
    ++g_bad;
  }
}

void run_codebook(std::istringstream& in) {
  int d = 0, bits = 0;
  in >> d >> bits;
  const int L = 1 << bits;
  std::vector<float> c(L), t(L - 1);
  int rc = hsq_codebook(d, bits, c.data(), t.data());
  std::printf("codebook %d", rc);
  for (float x : c) std::printf(" %.9g", x);
  std::printf(" |");
  for (float x : t) std::printf(" %.9g", x);
  std::printf("\n");
}

void run_tier(std::istringstream& in) {
  int T = 0, ns = 0, nr = 0, gn = 0, nm = 0;
  in >> T >> ns >> nr >> gn >> nm;
  std::vector<int32_t> marked(nm);
  for (int i = 0; i < nm; ++i) in >> marked[i];
  const int32_t* mp = nm ? marked.data() : nullptr;
  int n1 = -1, ng = -1;
  int rc = hsq_tier_plan(T, ns, nr, mp, nm, gn, nullptr, &n1, nullptr, &ng);
  if (rc) {
    std::printf("tier %d\n", rc);
    return;
  }
  // exact-size outputs: the second call must write n1 and ng * gn entries only
  std::vector<int32_t> l1(n1), gp((size_t)ng * gn);
  int n1b = -1, ngb = -1;
  rc = hsq_tier_plan(T, ns, nr, mp, nm, gn, l1.data(), &n1b, gp.data(), &ngb);
  if (rc || n1b != n1 || ngb != ng) {
    std::printf("tier %d counts differ between calls\n", rc ? rc : -100);
    return;
  }
  std::printf("tier %d %d %d |", rc, n1, ng);
  for (int x : l1) std::printf(" %d", x);
  std::printf(" |");
  for (int x : gp) std::printf(" %d", x);
  std::printf("\n");
}

void run_workspace(std::istringstream& in) {
  int B, Hq, Hkv, d, n1, ng, beta, gn;
  in >> B >> Hq >> Hkv >> d >> n1 >> ng >> beta >> gn;
  std::printf("workspace %zu\n", hsq_workspace_bytes(B, Hq, Hkv, d, n1, ng, beta, gn));
}

// Every call below fails validation, so no pointer is dereferenced.
void run_errors() {
  void* p = reinterpret_cast<void*>(16);
  const auto u8 = static_cast<uint8_t*>(p);
  const auto f32 = static_cast<float*>(p);
  const auto i32 = static_cast<int32_t*>(p);
  const auto u32 = static_cast<uint32_t*>(p);
  float c[16];
  expect("codebook d=2", hsq_codebook(2, 4, c, c), HSQ_ERR_ARG);
  expect("codebook bits=5", hsq_codebook(64, 5, c, c), HSQ_ERR_ARG);
  expect("codebook null", hsq_codebook(64, 4, nullptr, c), HSQ_ERR_ARG, "null");

  // encode / decode: unsupported d, bits, dtype; sizes; null pointers
  expect("encode d=96", hsq_encode(p, 0, 10, 96, 4, nullptr, 1, u32, 1, 1, f32, u8, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("encode bits=1", hsq_encode(p, 0, 10, 128, 1, nullptr, 1, u32, 1, 1, f32, u8, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("encode bits=5", hsq_encode(p, 0, 10, 128, 5, nullptr, 1, u32, 1, 1, f32, u8, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("decode bits=1", hsq_decode(u8, f32, 10, 128, 1, nullptr, 1, 1, f32, p, 0, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("decode bits=5", hsq_decode(u8, f32, 10, 128, 5, nullptr, 1, 1, f32, p, 0, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("encode 2^32", hsq_encode(p, 0, int64_t(1) << 32, 128, 4, nullptr, 1, u32, 1, 1, f32, u8,
                                   f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("decode 2^32", hsq_decode(u8, f32, int64_t(1) << 32, 128, 4, u32, 1, 1, f32, p, 0, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("build_tiers rows", hsq_build_tiers(p, p, 0, 1 << 16, 1 << 8, 1 << 8, 128, i32, 16, i32, 4,
                                             8, u32, u32, f32, f32, u8, f32, u8, f32, u8, f32, u8,
                                             f32, u8, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("build_tiers n1+ng*N>T", hsq_build_tiers(p, p, 0, 1, 1, 40, 128, i32, 16, i32, 4, 8, u32,
                                                  u32, f32, f32, u8, f32, u8, f32, u8, f32, u8,
                                                  f32, u8, nullptr),
         HSQ_ERR_ARG);
  expect("build_tiers null L3", hsq_build_tiers(p, p, 0, 1, 1, 64, 128, i32, 16, i32, 4, 8, u32,
                                                u32, f32, f32, u8, f32, u8, f32, u8, f32, u8, f32,
                                                nullptr, nullptr),
         HSQ_ERR_ARG, "null");
  expect("encode null thr", hsq_encode(p, 0, 10, 128, 2, nullptr, 1, nullptr, 1, 1, nullptr, u8,
                                       f32, nullptr),
         HSQ_ERR_ARG);
  expect("decode null cb", hsq_decode(u8, f32, 10, 128, 2, nullptr, 1, 1, nullptr, p, 0, nullptr),
         HSQ_ERR_ARG);
  expect("encode dtype=7", hsq_encode(p, 7, 10, 128, 4, nullptr, 1, u32, 1, 1, f32, u8, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("encode null x", hsq_encode(nullptr, 0, 10, 128, 4, nullptr, 1, u32, 1, 1, f32, u8, f32,
                                     nullptr),
         HSQ_ERR_ARG);
  expect("encode n<0", hsq_encode(p, 0, -1, 128, 4, nullptr, 1, u32, 1, 1, f32, u8, f32, nullptr),
         HSQ_ERR_ARG);
  expect("encode group_n=0", hsq_encode(p, 0, 10, 128, 4, nullptr, 0, u32, 1, 1, f32, u8, f32,
                                        nullptr),
         HSQ_ERR_ARG);
  expect("encode empty", hsq_encode(nullptr, 0, 0, 128, 4, nullptr, 1, nullptr, 1, 1, nullptr,
                                    nullptr, nullptr, nullptr),
         HSQ_OK);
  expect("decode_rope base", hsq_decode_rope(u8, f32, 10, 128, 4, u32, 1, 1, f32, i32, -2.0, p, 0,
                                             nullptr),
         HSQ_ERR_ARG, "rope_base");
  expect("decode_rope null pos", hsq_decode_rope(u8, f32, 10, 128, 4, u32, 1, 1, f32, nullptr, 1e6,
                                                 p, 0, nullptr),
         HSQ_ERR_ARG, "null");

  // decode-step shapes: Hq % Hkv, G > 8, group size, beta < 0, workspace
  expect("workspace Hq%Hkv", (long)hsq_workspace_bytes(1, 10, 4, 128, 10, 10, 2, 16), 0);
  expect("workspace G=9", (long)hsq_workspace_bytes(1, 36, 4, 128, 10, 10, 2, 16), 0);
  expect("workspace N=12", (long)hsq_workspace_bytes(1, 32, 8, 128, 10, 10, 2, 12), 0);
  expect("workspace beta<0", (long)hsq_workspace_bytes(1, 32, 8, 128, 10, 10, -1, 16), 0);
  expect("route no workspace", hsq_route_topk(f32, 1, 32, 8, 128, u8, f32, 10, u32, f32, 0.1f, 0,
                                              2, i32, nullptr, nullptr, 0, nullptr),
         HSQ_ERR_WORKSPACE);
  expect("route agg=9", hsq_route_topk(f32, 1, 32, 8, 128, u8, f32, 10, u32, f32, 0.1f, 9, 2, i32,
                                       nullptr, nullptr, 0, nullptr),
         HSQ_ERR_ARG);
  const size_t ws = hsq_workspace_bytes(2, 32, 8, 128, 40, 30, 4, 16);
  expect("step no workspace", hsq_decode_step(f32, 2, 32, 8, 128, u8, f32, u8, f32, 40, u8, f32, u8,
                                              f32, 30, u8, 16, 4, 0, u32, u32, f32, f32, 0.1f,
                                              0.f, i32, nullptr, ws, f32, nullptr),
         HSQ_ERR_WORKSPACE);
  expect("step small workspace", hsq_decode_step(f32, 2, 32, 8, 128, u8, f32, u8, f32, 40, u8, f32,
                                                 u8, f32, 30, u8, 16, 4, 0, u32, u32, f32, f32,
                                                 0.1f, 0.f, i32, p, ws - 1, f32, nullptr),
         HSQ_ERR_WORKSPACE);
  expect("step unaligned workspace", hsq_decode_step(f32, 2, 32, 8, 128, u8, f32, u8, f32, 40, u8,
                                                     f32, u8, f32, 30, u8, 16, 4, 0,
                                                     u32, u32, f32, f32, 0.1f, 0.f, i32,
                                                     reinterpret_cast<void*>(4096 + 16), ws, f32,
                                                     nullptr),
         HSQ_ERR_ARG, "aligned");
  expect("step agg=3", hsq_decode_step(f32, 2, 32, 8, 128, u8, f32, u8, f32, 40, u8, f32, u8, f32,
                                       30, u8, 16, 4, 3, u32, u32, f32, f32, 0.1f, 0.f, i32, p, ws,
                                       f32, nullptr),
         HSQ_ERR_ARG);
  expect("step null L3", hsq_decode_step(f32, 2, 32, 8, 128, u8, f32, u8, f32, 40, u8, f32, u8,
                                         f32, 30, nullptr, 16, 4, 0, u32, u32, f32, f32, 0.1f, 0.f,
                                         i32, p, ws, f32, nullptr),
         HSQ_ERR_ARG, "null");
  expect("step too many groups", hsq_decode_step(f32, 1, 8, 8, 128, u8, f32, u8, f32, 40, u8, f32,
                                                 u8, f32, 1 << 20, u8, 16, 4, 0, u32, u32, f32,
                                                 f32, 0.1f, 0.f, i32, p, size_t(1) << 40, f32,
                                                 nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("step_static too large", hsq_decode_step_static(f32, 64, 64, 8, 128, u8, f32, u8, f32,
                                                         40, u8, f32, u8, f32, 16000, u8, 16, 500,
                                                         0, u32, u32, f32, f32, 0.1f, 0.f, i32,
                                                         f32, nullptr),
         HSQ_ERR_UNSUPPORTED, "scratch");
  expect("attn beta>ng", hsq_decode_attn(f32, 1, 8, 8, 128, u8, f32, u8, f32, 40, u8, f32, u8, f32,
                                         3, u8, 16, 0, i32, 4, u32, u32, f32, f32, 0.1f, 0.f, p,
                                         ws, f32, nullptr),
         HSQ_ERR_ARG);
  expect("step_route null q", hsq_step_route(nullptr, 1, 8, 8, 128, 40, u8, f32, u8, f32, 3, 16, 2,
                                             0, u32, f32, 0.1f, 0.f, i32, p, ws, nullptr),
         HSQ_ERR_ARG, "null");
  expect("step_attend null L1", hsq_step_attend(f32, 1, 8, 8, 128, nullptr, f32, u8, f32, 40, 3,
                                                u8, 16, 0, 2, u32, u32, f32, 0.1f, p, ws, f32,
                                                nullptr),
         HSQ_ERR_ARG, "L1");
  expect("gather rec_bytes", hsq_gather_l3(u8, 100, 1, 1, 4, i32, 2, u8, nullptr), HSQ_ERR_ARG);
  expect("gather beta>ng", hsq_gather_l3(u8, 1088, 1, 1, 4, i32, 5, u8, nullptr), HSQ_ERR_ARG);
  expect("gather rec > 1 MiB", hsq_gather_l3(u8, (1u << 20) + 16, 1, 1, 4, i32, 2, u8, nullptr),
         HSQ_ERR_UNSUPPORTED, "1 MiB");
  expect("ordered gather null turn",
         hsq_gather_l3_ordered(u8, 1088, 1, 1, 4, i32, 2, u8, nullptr, 0u, nullptr), HSQ_ERR_ARG,
         "turn");
  expect("ordered gather misaligned turn",
         hsq_gather_l3_ordered(u8, 1088, 1, 1, 4, i32, 2, u8, reinterpret_cast<uint32_t*>(18), 0u,
                               nullptr),
         HSQ_ERR_ARG, "aligned");
  expect("ordered gather beta>ng", hsq_gather_l3_ordered(u8, 1088, 1, 1, 4, i32, 5, u8, u32, 0u,
                                                         nullptr),
         HSQ_ERR_ARG);
  expect("tier_plan null marks", hsq_tier_plan(10, 1, 1, nullptr, 3, 8, nullptr, nullptr, nullptr,
                                               nullptr),
         HSQ_ERR_ARG);
  int n1 = 0, ng = 0;
  int32_t bad_mark = 10;
  expect("tier_plan mark>=T", hsq_tier_plan(10, 1, 1, &bad_mark, 1, 8, nullptr, &n1, nullptr, &ng),
         HSQ_ERR_ARG, "range");
  expect("tier_plan T=0", hsq_tier_plan(0, 1, 1, nullptr, 0, 8, nullptr, &n1, nullptr, &ng),
         HSQ_ERR_ARG);

  // decode-time cache
  void* P[16];
  for (auto& x : P) x = p;
  auto app = [&](int dtype, int d, int N, int64_t t, int pend, int ng_, int l1_cap, int ng_cap,
                 int null_at) {
    void* a[16];
    std::memcpy(a, P, sizeof a);
    if (null_at >= 0) a[null_at] = nullptr;
    return hsq_cache_append(p, p, dtype, 1, 1, d, N, 4, 16, t, pend, ng_, l1_cap, ng_cap,
                            (uint32_t*)a[0], (uint32_t*)a[1], (float*)a[2], (float*)a[3],
                            (uint8_t*)a[4], (float*)a[5], (uint8_t*)a[6], (float*)a[7], a[8],
                            a[9], (uint8_t*)a[10], (float*)a[11], (uint8_t*)a[12], (float*)a[13],
                            (uint8_t*)a[14], nullptr);
  };
  expect("append d=96", app(0, 96, 8, 100, 0, 3, 28, 10, -1), HSQ_ERR_UNSUPPORTED);
  expect("append N=12", app(0, 128, 12, 100, 0, 3, 28, 10, -1), HSQ_ERR_UNSUPPORTED);
  expect("append dtype=5", app(5, 128, 8, 100, 0, 3, 28, 10, -1), HSQ_ERR_UNSUPPORTED);
  expect("append window", app(0, 128, 8, 15, 0, 3, 28, 10, -1), HSQ_ERR_ARG);
  expect("append pending", app(0, 128, 8, 100, 8, 3, 28, 10, -1), HSQ_ERR_ARG);
  expect("append l1_cap", app(0, 128, 8, 100, 0, 3, 27, 10, -1), HSQ_ERR_ARG);
  expect("append seal full", app(0, 128, 8, 100, 7, 10, 28, 10, -1), HSQ_ERR_ARG);
  expect("append ng>cap", app(0, 128, 8, 100, 0, 11, 28, 10, -1), HSQ_ERR_ARG);
  expect("append null", app(0, 128, 8, 100, 0, 3, 28, 10, 10), HSQ_ERR_ARG, "null");
  auto cstep = [&](int n_l1, int l1_cap, int ng_, int ng_cap, int G, void* w) {
    return hsq_cache_decode_step(f32, 1, 8 * G, 8, 128, u8, f32, u8, f32, n_l1, l1_cap, u8, f32,
                                 u8, f32, ng_, ng_cap, u8, 8, 2, 0, u32, u32, f32, f32, 0.1f,
                                 0.f, nullptr, w, 0, f32, nullptr);
  };
  expect("cache step l1_cap", cstep(20, 19, 3, 10, 4, p), HSQ_ERR_ARG);
  expect("cache step ng_cap", cstep(20, 28, 3, 2, 4, p), HSQ_ERR_ARG);
  expect("cache step G=9", cstep(20, 28, 3, 10, 9, p), HSQ_ERR_UNSUPPORTED);
  expect("cache step no workspace", cstep(20, 28, 3, 10, 4, nullptr), HSQ_ERR_WORKSPACE);

  // QJL
  expect("qjl d=96", hsq_encode_qjl(p, 0, 10, 96, 4, u32, f32, f32, f32, u8, f32, u8, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("qjl bits=2", hsq_encode_qjl(p, 0, 10, 128, 2, u32, f32, f32, f32, u8, f32, u8, f32,
                                      nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("qjl null", hsq_encode_qjl(p, 0, 10, 128, 4, u32, f32, f32, f32, nullptr, f32, u8, f32,
                                    nullptr),
         HSQ_ERR_ARG, "null");
  expect("qjl empty", hsq_encode_qjl(nullptr, 0, 0, 128, 4, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, nullptr),
         HSQ_OK);
  expect("qjl logits n_q=9", hsq_qjl_logits(f32, 9, 128, 4, u8, f32, u8, f32, 10, u32, f32, f32,
                                            0.1f, f32, nullptr),
         HSQ_ERR_ARG);
  expect("qjl logits d=32", hsq_qjl_logits(f32, 4, 32, 4, u8, f32, u8, f32, 10, u32, f32, f32,
                                           0.1f, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);

  // pre-RoPE and TQ-QKV steps, sketch build
  const size_t plain = hsq_workspace_bytes(2, 32, 8, 128, 10, 10, 4, 16);
  const size_t pre = hsq_prerope_workspace_bytes(2, 32, 8, 128, 10, 10, 4, 16);
  expect("prerope workspace size", pre >= plain + size_t(2) * 8 * 4 * 16 * 128 * 2 ? 0 : 1, 0);
  void* wsa = reinterpret_cast<void*>(256);
  auto prestep = [&](const int32_t* pos, double base, size_t wb) {
    return hsq_decode_step_prerope(f32, 2, 32, 8, 128, u8, f32, u8, f32, 10, u8, f32, u8, f32, 10,
                                   u8, 16, 4, 0, u32, u32, f32, f32, 0.1f, 0.f, pos, base, nullptr,
                                   wsa, wb, f32, nullptr);
  };
  expect("prerope null positions", prestep(nullptr, 1e6, pre), HSQ_ERR_ARG, "group_pos");
  expect("prerope base 0", prestep(i32, 0.0, pre), HSQ_ERR_ARG, "rope_base");
  expect("prerope small workspace", prestep(i32, 1e6, plain), HSQ_ERR_WORKSPACE);
  auto qstep = [&](const uint8_t* l1s, const float* l3g, const float* S) {
    return hsq_decode_step_qjl(f32, 2, 32, 8, 128, u8, f32, u8, f32, 10, u8, f32, u8, f32, 10, u8,
                               16, 4, 0, u32, u32, f32, f32, 0.1f, 0.f, l1s, f32, u8, l3g, S,
                               nullptr, wsa, plain, f32, nullptr);
  };
  expect("qjl step null S", qstep(u8, f32, nullptr), HSQ_ERR_ARG, "S");
  expect("qjl step null L1 sketch", qstep(nullptr, f32, f32), HSQ_ERR_ARG, "L1");
  expect("qjl step null archive gamma", qstep(u8, nullptr, f32), HSQ_ERR_ARG, "archive");
  expect("sketches n1+ng*N>T", hsq_build_sketches(p, 0, 1, 1, 40, 128, i32, 16, i32, 4, 8, u32,
                                                   f32, f32, f32, u8, f32, u8, f32, nullptr),
         HSQ_ERR_ARG);
  expect("sketches d=96", hsq_build_sketches(p, 0, 1, 1, 64, 96, i32, 16, i32, 4, 8, u32, f32,
                                              f32, f32, u8, f32, u8, f32, nullptr),
         HSQ_ERR_UNSUPPORTED);
  expect("sketches null S", hsq_build_sketches(p, 0, 1, 1, 64, 128, i32, 16, i32, 4, 8, u32, f32,
                                                f32, nullptr, u8, f32, u8, f32, nullptr),
         HSQ_ERR_ARG, "null");
  std::printf("errors %d\n", g_checked);
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "codebook") run_codebook(in);
    else if (cmd == "tier") run_tier(in);
    else if (cmd == "workspace") run_workspace(in);
    else if (cmd == "errors") run_errors();
    else {
      std::fprintf(stderr, "unknown command %s\n", cmd.c_str());
      return 2;
    }
  }
  std::fflush(stdout);
  return g_bad ? 1 : 0;
}
