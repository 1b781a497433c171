// C ABI of libhsq: argument validation, error reporting and launches.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "hsq_internal.h"

namespace hsq {

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return HSQ_OK;
  return fail(HSQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace hsq

using namespace hsq;

namespace {

bool supported_d(int d) { return d == 64 || d == 128; }
bool supported_bits(int b) { return b == 3 || b == 4; }
bool codec_bits(int b) { return b >= 2 && b <= 4; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int check_step_shape(const char* fn, int B, int Hq, int Hkv, int d, int n_l1, int n_groups,
                     int group_n, int beta) {
  if (B < 1 || Hq < 1 || Hkv < 1 || n_l1 < 0 || n_groups < 0 || beta < 0)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": sizes must be positive (n_l1, n_groups, beta >= 0)");
  if (Hq % Hkv) return fail(HSQ_ERR_ARG, std::string(fn) + ": Hq must be a multiple of Hkv");
  if (Hq / Hkv > 8) return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": at most 8 query heads per kv-head");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": d must be 64 or 128");
  if (group_n != 8 && group_n != 16)
    return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": group_n must be 8 or 16");
  return HSQ_OK;
}

}  // namespace

extern "C" const char* hsq_version(void) { return "hsq 0.1 gfx950"; }
extern "C" const char* hsq_last_error(void) { return g_last_error.c_str(); }

extern "C" int hsq_encode(const void* x, int x_dtype, int64_t n_vec, int d, int bits,
                          const int64_t* row_idx, int group_n, const uint32_t* signs,
                          int64_t vecs_per_rot, int n_rot, const float* thresholds,
                          uint8_t* codes, float* norms, void* stream) {
  if (n_vec < 0 || group_n < 1 || vecs_per_rot < 1 || n_rot < 1)
    return fail(HSQ_ERR_ARG, "hsq_encode: bad sizes");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode: d must be 64 or 128");
  if (!codec_bits(bits)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode: bits must be 2, 3 or 4");
  if (x_dtype != HSQ_F32 && x_dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode: x_dtype must be HSQ_F32 or HSQ_BF16");
  if (n_vec > (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode: at most 2^32 - 1 vectors per call");
  if (n_vec == 0) return HSQ_OK;
  if (!x || !thresholds || !codes || !norms)  // signs may be null: rotation off
    return fail(HSQ_ERR_ARG, "hsq_encode: null pointer");
  EncodeJob j{};
  j.x = x; j.dtype = x_dtype; j.n_vec = n_vec; j.d = d; j.bits = bits; j.group_n = group_n;
  j.row_idx = row_idx;
  j.signs = signs; j.vecs_per_rot = vecs_per_rot; j.n_rot = n_rot; j.thr = thresholds;
  j.codes = codes; j.code_rec_bytes = d * bits / 8; j.norms = norms; j.norm_rec_floats = 1;
  j.vecs_per_rec = 1;
  return check_hip(launch_encode(j, as_stream(stream)), "hsq_encode launch");
}

extern "C" int hsq_decode(const uint8_t* codes, const float* norms, int64_t n_vec, int d, int bits,
                          const uint32_t* signs, int64_t vecs_per_rot, int n_rot,
                          const float* centroids, void* out, int out_dtype, void* stream) {
  if (n_vec < 0 || vecs_per_rot < 1 || n_rot < 1) return fail(HSQ_ERR_ARG, "hsq_decode: bad sizes");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode: d must be 64 or 128");
  if (!codec_bits(bits)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode: bits must be 2, 3 or 4");
  if (out_dtype != HSQ_F32 && out_dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode: out_dtype must be HSQ_F32 or HSQ_BF16");
  if (n_vec > (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode: at most 2^32 - 1 vectors per call");
  if (n_vec == 0) return HSQ_OK;
  if (!codes || !norms || !centroids || !out)  // signs may be null: rotation off
    return fail(HSQ_ERR_ARG, "hsq_decode: null pointer");
  DecodeJob j{codes, norms, n_vec, d, bits, signs, vecs_per_rot, n_rot, centroids, out, out_dtype};
  return check_hip(launch_decode(j, as_stream(stream)), "hsq_decode launch");
}

extern "C" int hsq_decode_rope(const uint8_t* codes, const float* norms, int64_t n_vec, int d,
                               int bits, const uint32_t* signs, int64_t vecs_per_rot, int n_rot,
                               const float* centroids, const int32_t* positions,
                               double rope_base, void* out, int out_dtype, void* stream) {
  if (n_vec < 0 || vecs_per_rot < 1 || n_rot < 1)
    return fail(HSQ_ERR_ARG, "hsq_decode_rope: bad sizes");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode_rope: d must be 64 or 128");
  if (!codec_bits(bits)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode_rope: bits must be 2, 3 or 4");
  if (out_dtype != HSQ_F32 && out_dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode_rope: out_dtype must be HSQ_F32 or HSQ_BF16");
  if (!(rope_base > 0.0) || !std::isfinite(rope_base))
    return fail(HSQ_ERR_ARG, "hsq_decode_rope: rope_base must be finite and positive");
  if (n_vec > (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_decode_rope: at most 2^32 - 1 vectors per call");
  if (n_vec == 0) return HSQ_OK;
  if (!codes || !norms || !centroids || !positions || !out)  // signs may be null: rotation off
    return fail(HSQ_ERR_ARG, "hsq_decode_rope: null pointer");
  DecodeJob j{codes, norms, n_vec, d, bits, signs, vecs_per_rot, n_rot, centroids, out, out_dtype,
              positions, rope_base};
  return check_hip(launch_decode(j, as_stream(stream)), "hsq_decode_rope launch");
}

extern "C" int hsq_build_tiers(const void* k, const void* v, int dtype, int B, int Hkv, int T,
                               int d, const int32_t* l1_pos, int n1, const int32_t* group_pos,
                               int n_groups, int group_n, const uint32_t* k_signs,
                               const uint32_t* v_signs, const float* thr4, const float* thr3,
                               uint8_t* l1k, float* l1k_n, uint8_t* l1v, float* l1v_n,
                               uint8_t* l2k, float* l2k_n, uint8_t* l2v, float* l2v_n,
                               uint8_t* l3, void* stream) {
  if (B < 1 || Hkv < 1 || T < 1 || n1 < 0 || n_groups < 0 || group_n < 1)
    return fail(HSQ_ERR_ARG, "hsq_build_tiers: bad sizes");
  if ((int64_t)B * Hkv * T > (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_build_tiers: at most 2^32 - 1 rows (B * Hkv * T)");
  if ((int64_t)n1 + (int64_t)n_groups * group_n > T)
    return fail(HSQ_ERR_ARG, "hsq_build_tiers: n1 + n_groups * group_n exceeds T");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_build_tiers: d must be 64 or 128");
  if (dtype != HSQ_F32 && dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_build_tiers: dtype must be HSQ_F32 or HSQ_BF16");
  if (!k || !v || !k_signs || !v_signs || !thr4 || !thr3)
    return fail(HSQ_ERR_ARG, "hsq_build_tiers: null input pointer");
  if (n1 > 0 && (!l1_pos || !l1k || !l1k_n || !l1v || !l1v_n))
    return fail(HSQ_ERR_ARG, "hsq_build_tiers: null L1 pointer");
  if (n_groups > 0 && (!group_pos || !l2k || !l2k_n || !l2v || !l2v_n || !l3))
    return fail(HSQ_ERR_ARG, "hsq_build_tiers: null L2/L3 pointer");
  const hipStream_t st = as_stream(stream);
  const int64_t units = (int64_t)B * Hkv;
  const int64_t cb4 = d / 2, cb3 = 3 * d / 8;
  for (int kv = 0; kv < 2; ++kv) {
    EncodeJob j{};
    j.x = kv ? v : k; j.dtype = dtype; j.d = d;
    j.units_per_seq = Hkv; j.rows_per_unit = T;
    j.signs = kv ? v_signs : k_signs; j.n_rot = Hkv;
    if (n1 > 0) {  // L1: one 4-bit vector per L1 position
      EncodeJob a = j;
      a.bits = 4; a.group_n = 1; a.n_vec = units * n1; a.pos = l1_pos; a.vecs_per_unit = n1;
      a.pos_per_seq = n1; a.vecs_per_rot = n1; a.thr = thr4;
      a.codes = kv ? l1v : l1k; a.code_rec_bytes = cb4; a.norms = kv ? l1v_n : l1k_n;
      a.norm_rec_floats = 1; a.vecs_per_rec = 1;
      int rc = check_hip(launch_encode(a, st), "hsq_build_tiers L1");
      if (rc) return rc;
    }
    if (n_groups > 0) {
      // L2: 3-bit code of the mean of each group's N raw vectors
      EncodeJob a = j;
      a.bits = 3; a.group_n = group_n; a.n_vec = units * n_groups; a.pos = group_pos;
      a.vecs_per_unit = n_groups; a.pos_per_seq = (int64_t)n_groups * group_n;
      a.vecs_per_rot = n_groups; a.thr = thr3;
      a.codes = kv ? l2v : l2k; a.code_rec_bytes = cb3; a.norms = kv ? l2v_n : l2k_n;
      a.norm_rec_floats = 1; a.vecs_per_rec = 1;
      int rc = check_hip(launch_encode(a, st), "hsq_build_tiers L2");
      if (rc) return rc;
      // L3: 4-bit code of every grouped token, written into group records
      EncodeJob c = j;
      const int64_t rec = (int64_t)group_n * (d + 8);
      c.bits = 4; c.group_n = 1; c.n_vec = units * n_groups * group_n; c.pos = group_pos;
      c.vecs_per_unit = (int64_t)n_groups * group_n; c.pos_per_seq = c.vecs_per_unit;
      c.vecs_per_rot = c.vecs_per_unit; c.thr = thr4;
      const int64_t base = kv ? group_n * (cb4 + 4) : 0;
      c.codes = l3 + base; c.code_rec_bytes = rec;
      c.norms = reinterpret_cast<float*>(l3 + base + group_n * cb4); c.norm_rec_floats = rec / 4;
      c.vecs_per_rec = group_n;
      rc = check_hip(launch_encode(c, st), "hsq_build_tiers L3");
      if (rc) return rc;
    }
  }
  return HSQ_OK;
}

extern "C" size_t hsq_workspace_bytes(int B, int Hq, int Hkv, int d, int n_l1, int n_groups,
                                      int beta, int group_n) {
  if (check_step_shape("hsq_workspace_bytes", B, Hq, Hkv, d, n_l1, n_groups, group_n, beta))
    return 0;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, beta < n_groups ? beta : n_groups};
  return plan_workspace(s).total;
}

namespace {

int step_common(const char* fn, const StepShape& s, void* workspace, size_t ws_bytes,
                Workspace& w) {
  if (!step_limits_ok(s))
    return fail(HSQ_ERR_UNSUPPORTED,
                std::string(fn) + ": n_groups or the L1/L3 sizes exceed the kernels' limits "
                                  "(n_groups <= 16384, per-unit L1/L3 bytes < 2 GiB)");
  w = plan_workspace(s);
  if (!workspace || ws_bytes < w.total)
    return fail(HSQ_ERR_WORKSPACE, std::string(fn) + ": workspace missing or smaller than hsq_workspace_bytes()");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": workspace must be 256-byte aligned");
  return HSQ_OK;
}

int need_route_lds(const char* fn, const StepShape& s) {
  if (s.n_groups > 0 && !route_lds_ok(s))
    return fail(HSQ_ERR_UNSUPPORTED,
                std::string(fn) + ": G * n_groups exceeds 12288 (the router logits this call "
                                  "holds on chip); hsq_decode_step serves such shapes");
  return HSQ_OK;
}

}  // namespace

extern "C" int hsq_route_topk(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l2k,
                              const float* l2k_n, int n_groups, const uint32_t* k_signs,
                              const float* cb3, float scale, int agg, int beta,
                              int32_t* topk_idx, float* scores, void* workspace,
                              size_t ws_bytes, void* stream) {
  int rc = check_step_shape("hsq_route_topk", B, Hq, Hkv, d, 0, n_groups, 8, beta);
  if (rc) return rc;
  if (agg != HSQ_AGG_MAX && agg != HSQ_AGG_MEAN) return fail(HSQ_ERR_ARG, "hsq_route_topk: bad agg");
  if (!q || !k_signs || !cb3 || (n_groups > 0 && (!l2k || !l2k_n)))
    return fail(HSQ_ERR_ARG, "hsq_route_topk: null input pointer");
  const int b = beta < n_groups ? beta : n_groups;
  if (b > 0 && !topk_idx) return fail(HSQ_ERR_ARG, "hsq_route_topk: null topk_idx");
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, 0, n_groups, 8, b};
  Workspace w;
  if ((rc = step_common("hsq_route_topk", s, workspace, ws_bytes, w))) return rc;
  if (n_groups == 0) return HSQ_OK;
  StepTensors t{};
  t.q = q; t.l2k = l2k; t.l2k_n = l2k_n; t.k_signs = k_signs; t.cb3 = cb3; t.scale = scale;
  t.agg = agg;
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = as_stream(stream);
  return check_hip(launch_route(s, t, w, ws, ROUTE_TOPK, nullptr, scores, topk_idx, st),
                   "hsq_route_topk route");
}

namespace {

int attn_args(const char* fn, const float* q, const uint8_t* l1k, const float* l1k_n,
              const uint8_t* l1v, const float* l1v_n, int n_l1, const uint8_t* l2k,
              const float* l2k_n, const uint8_t* l2v, const float* l2v_n, int n_groups,
              const uint8_t* l3, const uint32_t* k_signs, const uint32_t* v_signs,
              const float* cb4, const float* cb3, float* out) {
  if (!q || !out || !k_signs || !v_signs || !cb4 || !cb3)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null pointer");
  if (n_l1 > 0 && (!l1k || !l1k_n || !l1v || !l1v_n))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null L1 pointer");
  if (n_groups > 0 && (!l2k || !l2k_n || !l2v || !l2v_n || !l3))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null L2/L3 pointer");
  return HSQ_OK;
}

}  // namespace

extern "C" int hsq_decode_attn(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                               const float* l1k_n, const uint8_t* l1v, const float* l1v_n,
                               int n_l1, const uint8_t* l2k, const float* l2k_n,
                               const uint8_t* l2v, const float* l2v_n, int n_groups,
                               const uint8_t* l3, int group_n, int l3_staged,
                               const int32_t* topk_idx, int beta, const uint32_t* k_signs,
                               const uint32_t* v_signs, const float* cb4, const float* cb3,
                               float scale, float summary_bias, void* workspace,
                               size_t ws_bytes, float* out, void* stream) {
  int rc = check_step_shape("hsq_decode_attn", B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if (beta > n_groups) return fail(HSQ_ERR_ARG, "hsq_decode_attn: beta exceeds n_groups");
  if ((rc = attn_args("hsq_decode_attn", q, l1k, l1k_n, l1v, l1v_n, n_l1, l2k, l2k_n, l2v, l2v_n,
                      n_groups, l3, k_signs, v_signs, cb4, cb3, out)))
    return rc;
  if (beta > 0 && !topk_idx) return fail(HSQ_ERR_ARG, "hsq_decode_attn: null topk_idx");
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, beta};
  Workspace w;
  if ((rc = step_common("hsq_decode_attn", s, workspace, ws_bytes, w))) return rc;
  if ((rc = need_route_lds("hsq_decode_attn", s))) return rc;
  StepTensors t{q, l1k, l1k_n, l1v, l1v_n, l2k, l2k_n, l2v, l2v_n, l3, l3_staged ? 1 : 0,
                k_signs, v_signs, cb4, cb3, scale, summary_bias, HSQ_AGG_MAX, out};
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = as_stream(stream);
  if ((rc = check_hip(launch_route(s, t, w, ws, ROUTE_PARTIALS, topk_idx, nullptr, nullptr, st),
                      "hsq_decode_attn summaries")))
    return rc;
  return check_hip(launch_attn(s, t, w, ws, topk_idx, st), "hsq_decode_attn attention");
}

extern "C" int hsq_step_route(const float* q, int B, int Hq, int Hkv, int d, int n_l1,
                              const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                              const float* l2v_n, int n_groups, int group_n, int beta, int agg,
                              const uint32_t* k_signs, const float* cb3, float scale,
                              float summary_bias, int32_t* topk_idx, void* workspace,
                              size_t ws_bytes, void* stream) {
  int rc = check_step_shape("hsq_step_route", B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if (agg != HSQ_AGG_MAX && agg != HSQ_AGG_MEAN) return fail(HSQ_ERR_ARG, "hsq_step_route: bad agg");
  if (!q || !k_signs || !cb3 || (n_groups > 0 && (!l2k || !l2k_n || !l2v || !l2v_n)))
    return fail(HSQ_ERR_ARG, "hsq_step_route: null pointer");
  const int b = beta < n_groups ? beta : n_groups;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  Workspace w;
  if ((rc = step_common("hsq_step_route", s, workspace, ws_bytes, w))) return rc;
  StepTensors t{};
  t.q = q; t.l2k = l2k; t.l2k_n = l2k_n; t.l2v = l2v; t.l2v_n = l2v_n; t.k_signs = k_signs;
  t.cb3 = cb3; t.scale = scale; t.summary_bias = summary_bias; t.agg = agg;
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = as_stream(stream);
  if (s.n_groups > 0 && !route_lds_ok(s))  // router logits beyond LDS: the split step's first half
    return check_hip(launch_split_half(s, t, w, ws, true, b > 0 ? topk_idx : nullptr, st),
                     "hsq_step_route (split)");
  if ((rc = need_route_lds("hsq_step_route", s))) return rc;
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx_off);
  if ((rc = check_hip(launch_route(s, t, w, ws, ROUTE_TOPK | ROUTE_PARTIALS, nullptr, nullptr,
                                   idx, st),
                      "hsq_step_route")))
    return rc;
  if (topk_idx && b > 0)
    return check_hip(hipMemcpyAsync(topk_idx, idx, sizeof(int32_t) * (size_t)B * Hkv * b,
                                    hipMemcpyDeviceToDevice, st),
                     "hsq_step_route topk copy");
  return HSQ_OK;
}

extern "C" int hsq_step_attend(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                               const float* l1k_n, const uint8_t* l1v, const float* l1v_n,
                               int n_l1, int n_groups, const uint8_t* l3, int group_n,
                               int l3_staged, int beta, const uint32_t* k_signs,
                               const uint32_t* v_signs, const float* cb4, float scale,
                               void* workspace, size_t ws_bytes, float* out, void* stream) {
  int rc = check_step_shape("hsq_step_attend", B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if (!q || !out || !k_signs || !v_signs || !cb4)
    return fail(HSQ_ERR_ARG, "hsq_step_attend: null pointer");
  if (n_l1 > 0 && (!l1k || !l1k_n || !l1v || !l1v_n))
    return fail(HSQ_ERR_ARG, "hsq_step_attend: null L1 pointer");
  const int b = beta < n_groups ? beta : n_groups;
  if (b > 0 && !l3) return fail(HSQ_ERR_ARG, "hsq_step_attend: null L3 pointer");
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  Workspace w;
  if ((rc = step_common("hsq_step_attend", s, workspace, ws_bytes, w))) return rc;
  StepTensors t{};
  t.q = q; t.l1k = l1k; t.l1k_n = l1k_n; t.l1v = l1v; t.l1v_n = l1v_n; t.l3 = l3;
  t.l3_staged = l3_staged ? 1 : 0; t.k_signs = k_signs; t.v_signs = v_signs; t.cb4 = cb4;
  t.scale = scale; t.out = out;
  char* ws = static_cast<char*>(workspace);
  if (s.n_groups > 0 && !route_lds_ok(s))  // the split step's second half, after hsq_step_route's
    return check_hip(launch_split_half(s, t, w, ws, false, nullptr, as_stream(stream)),
                     "hsq_step_attend (split)");
  if ((rc = need_route_lds("hsq_step_attend", s))) return rc;
  return check_hip(launch_attn(s, t, w, ws, reinterpret_cast<int32_t*>(ws + w.idx_off),
                               as_stream(stream)),
                   "hsq_step_attend");
}

extern "C" int hsq_decode_step(const float* q, int B, int Hq, int Hkv, int d, const uint8_t* l1k,
                               const float* l1k_n, const uint8_t* l1v, const float* l1v_n,
                               int n_l1, const uint8_t* l2k, const float* l2k_n,
                               const uint8_t* l2v, const float* l2v_n, int n_groups,
                               const uint8_t* l3, int group_n, int beta, int agg,
                               const uint32_t* k_signs, const uint32_t* v_signs,
                               const float* cb4, const float* cb3, float scale,
                               float summary_bias, int32_t* topk_idx, void* workspace,
                               size_t ws_bytes, float* out, void* stream) {
  int rc = check_step_shape("hsq_decode_step", B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if ((rc = attn_args("hsq_decode_step", q, l1k, l1k_n, l1v, l1v_n, n_l1, l2k, l2k_n, l2v, l2v_n,
                      n_groups, l3, k_signs, v_signs, cb4, cb3, out)))
    return rc;
  if (agg != HSQ_AGG_MAX && agg != HSQ_AGG_MEAN) return fail(HSQ_ERR_ARG, "hsq_decode_step: bad agg");
  const int b = beta < n_groups ? beta : n_groups;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  Workspace w;
  if ((rc = step_common("hsq_decode_step", s, workspace, ws_bytes, w))) return rc;
  StepTensors t{};
  t.q = q; t.l1k = l1k; t.l1k_n = l1k_n; t.l1v = l1v; t.l1v_n = l1v_n;
  t.l2k = l2k; t.l2k_n = l2k_n; t.l2v = l2v; t.l2v_n = l2v_n; t.l3 = l3; t.l3_staged = 0;
  t.k_signs = k_signs; t.v_signs = v_signs; t.cb4 = cb4; t.cb3 = cb3; t.scale = scale;
  t.summary_bias = summary_bias; t.agg = agg; t.out = out;
  if (use_split(s))  // beyond the one-launch step: each unit over many work-groups
    return check_hip(launch_split_step(s, t, w, static_cast<char*>(workspace),
                                       b > 0 ? topk_idx : nullptr, as_stream(stream)),
                     "hsq_decode_step (split)");
  if (step_fused_ok(s))  // one launch: route and attend on the same work-group
    return check_hip(launch_step(s, t, b > 0 ? topk_idx : nullptr, as_stream(stream)),
                     "hsq_decode_step");
  if ((rc = hsq_step_route(q, B, Hq, Hkv, d, n_l1, l2k, l2k_n, l2v, l2v_n, n_groups, group_n, beta,
                           agg, k_signs, cb3, scale, summary_bias, topk_idx, workspace, ws_bytes,
                           stream)))
    return rc;
  return hsq_step_attend(q, B, Hq, Hkv, d, l1k, l1k_n, l1v, l1v_n, n_l1, n_groups, l3, group_n, 0,
                         beta, k_signs, v_signs, cb4, scale, workspace, ws_bytes, out, stream);
}

namespace {

// fp16 fetched-key rows of the pre-RoPE step, after the step's own workspace
size_t prerope_rows_off(const Workspace& w) { return (w.total + 255) / 256 * 256; }
size_t prerope_rows_bytes(const StepShape& s) {
  return (size_t)s.B * s.Hkv * s.beta * s.group_n * s.d * 2;
}

}  // namespace

extern "C" size_t hsq_prerope_workspace_bytes(int B, int Hq, int Hkv, int d, int n_l1,
                                              int n_groups, int beta, int group_n) {
  if (check_step_shape("hsq_prerope_workspace_bytes", B, Hq, Hkv, d, n_l1, n_groups, group_n,
                       beta))
    return 0;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, beta < n_groups ? beta : n_groups};
  return prerope_rows_off(plan_workspace(s)) + prerope_rows_bytes(s);
}

extern "C" int hsq_step_attend_prerope(const float* q, int B, int Hq, int Hkv, int d,
                                       const uint8_t* l1k, const float* l1k_n,
                                       const uint8_t* l1v, const float* l1v_n, int n_l1,
                                       int n_groups, const uint8_t* l3, int group_n,
                                       int l3_staged, int beta, const uint32_t* k_signs,
                                       const uint32_t* v_signs, const float* cb4, float scale,
                                       const int32_t* group_pos, double rope_base,
                                       void* workspace, size_t ws_bytes, float* out,
                                       void* stream) {
  const char* fn = "hsq_step_attend_prerope";
  int rc = check_step_shape(fn, B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if (!q || !out || !k_signs || !v_signs || !cb4)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null pointer");
  if (n_l1 > 0 && (!l1k || !l1k_n || !l1v || !l1v_n))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null L1 pointer");
  const int b = beta < n_groups ? beta : n_groups;
  if (b > 0 && !l3) return fail(HSQ_ERR_ARG, std::string(fn) + ": null L3 pointer");
  if (n_groups > 0 && !group_pos) return fail(HSQ_ERR_ARG, std::string(fn) + ": null group_pos");
  if (!(rope_base > 0.0) || !std::isfinite(rope_base))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": rope_base must be finite and > 0");
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  Workspace w;
  if ((rc = step_common(fn, s, workspace, ws_bytes, w))) return rc;
  const size_t kd_off = prerope_rows_off(w);
  if (ws_bytes < kd_off + prerope_rows_bytes(s))
    return fail(HSQ_ERR_WORKSPACE,
                std::string(fn) + ": workspace smaller than hsq_prerope_workspace_bytes()");
  StepTensors t{};
  t.q = q; t.l1k = l1k; t.l1k_n = l1k_n; t.l1v = l1v; t.l1v_n = l1v_n; t.l3 = l3;
  t.l3_staged = l3_staged ? 1 : 0; t.k_signs = k_signs; t.v_signs = v_signs; t.cb4 = cb4;
  t.scale = scale; t.out = out;
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = as_stream(stream);
  const int32_t* idx = reinterpret_cast<const int32_t*>(ws + w.idx_off);
  uint16_t* rows = reinterpret_cast<uint16_t*>(ws + kd_off);
  if (b > 0) {
    RopeKeysJob j{};
    j.l3 = l3; j.unit_recs = n_groups; j.idx = idx; j.group_pos = group_pos;
    j.pos_per_seq = (int64_t)n_groups * group_n; j.units = B * Hkv; j.Hkv = Hkv; j.d = d;
    j.n_groups = n_groups; j.group_n = group_n; j.beta = b; j.k_signs = k_signs; j.cb4 = cb4;
    j.rope_base = rope_base; j.out = rows; j.staged = t.l3_staged;
    if ((rc = check_hip(launch_rope_keys(j, st), "hsq_step_attend_prerope fetched keys")))
      return rc;
  }
  if (s.n_groups > 0 && !route_lds_ok(s))  // the split step's second half, after its first
    return check_hip(launch_split_half(s, t, w, ws, false, nullptr, st, b > 0 ? rows : nullptr),
                     "hsq_step_attend_prerope (split)");
  return check_hip(launch_attn_prerope(s, t, w, ws, idx, b > 0 ? rows : nullptr, st),
                   "hsq_step_attend_prerope attention");
}

extern "C" int hsq_decode_step_prerope(const float* q, int B, int Hq, int Hkv, int d,
                                       const uint8_t* l1k, const float* l1k_n, const uint8_t* l1v,
                                       const float* l1v_n, int n_l1, const uint8_t* l2k,
                                       const float* l2k_n, const uint8_t* l2v, const float* l2v_n,
                                       int n_groups, const uint8_t* l3, int group_n, int beta,
                                       int agg, const uint32_t* k_signs, const uint32_t* v_signs,
                                       const float* cb4, const float* cb3, float scale,
                                       float summary_bias, const int32_t* group_pos,
                                       double rope_base, int32_t* topk_idx, void* workspace,
                                       size_t ws_bytes, float* out, void* stream) {
  const char* fn = "hsq_decode_step_prerope";
  int rc = check_step_shape(fn, B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if ((rc = attn_args(fn, q, l1k, l1k_n, l1v, l1v_n, n_l1, l2k, l2k_n, l2v, l2v_n, n_groups, l3,
                      k_signs, v_signs, cb4, cb3, out)))
    return rc;
  if (agg != HSQ_AGG_MAX && agg != HSQ_AGG_MEAN) return fail(HSQ_ERR_ARG, std::string(fn) + ": bad agg");
  if (n_groups > 0 && !group_pos) return fail(HSQ_ERR_ARG, std::string(fn) + ": null group_pos");
  if (!(rope_base > 0.0) || !std::isfinite(rope_base))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": rope_base must be finite and > 0");
  const int b = beta < n_groups ? beta : n_groups;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  Workspace w;
  if ((rc = step_common(fn, s, workspace, ws_bytes, w))) return rc;
  if (ws_bytes < prerope_rows_off(w) + prerope_rows_bytes(s))
    return fail(HSQ_ERR_WORKSPACE,
                std::string(fn) + ": workspace smaller than hsq_prerope_workspace_bytes()");
  // the route of the two-launch form (selection and summary partials into
  // the workspace), then the pre-RoPE attend over the archive in place
  if ((rc = hsq_step_route(q, B, Hq, Hkv, d, n_l1, l2k, l2k_n, l2v, l2v_n, n_groups, group_n, beta,
                           agg, k_signs, cb3, scale, summary_bias, topk_idx, workspace, ws_bytes,
                           stream)))
    return rc;
  return hsq_step_attend_prerope(q, B, Hq, Hkv, d, l1k, l1k_n, l1v, l1v_n, n_l1, n_groups, l3,
                                 group_n, 0, beta, k_signs, v_signs, cb4, scale, group_pos,
                                 rope_base, workspace, ws_bytes, out, stream);
}

extern "C" int hsq_decode_step_qjl(const float* q, int B, int Hq, int Hkv, int d,
                                   const uint8_t* l1k, const float* l1k_n, const uint8_t* l1v,
                                   const float* l1v_n, int n_l1, const uint8_t* l2k,
                                   const float* l2k_n, const uint8_t* l2v, const float* l2v_n,
                                   int n_groups, const uint8_t* l3, int group_n, int beta, int agg,
                                   const uint32_t* k_signs, const uint32_t* v_signs,
                                   const float* cb4, const float* cb3, float scale,
                                   float summary_bias, const uint8_t* l1_sketch,
                                   const float* l1_gamma, const uint8_t* l3_sketch,
                                   const float* l3_gamma, const float* S, int32_t* topk_idx,
                                   void* workspace, size_t ws_bytes, float* out, void* stream) {
  const char* fn = "hsq_decode_step_qjl";
  int rc = check_step_shape(fn, B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if ((rc = attn_args(fn, q, l1k, l1k_n, l1v, l1v_n, n_l1, l2k, l2k_n, l2v, l2v_n, n_groups, l3,
                      k_signs, v_signs, cb4, cb3, out)))
    return rc;
  if (agg != HSQ_AGG_MAX && agg != HSQ_AGG_MEAN) return fail(HSQ_ERR_ARG, std::string(fn) + ": bad agg");
  if (!S) return fail(HSQ_ERR_ARG, std::string(fn) + ": null S");
  if (n_l1 > 0 && (!l1_sketch || !l1_gamma))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null L1 sketch or gamma");
  if (n_groups > 0 && (!l3_sketch || !l3_gamma))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null archive sketch or gamma");
  if (reinterpret_cast<uintptr_t>(S) % 16 || reinterpret_cast<uintptr_t>(l1_sketch) % 4 ||
      reinterpret_cast<uintptr_t>(l3_sketch) % 4 || reinterpret_cast<uintptr_t>(l1_gamma) % 4 ||
      reinterpret_cast<uintptr_t>(l3_gamma) % 4)
    return fail(HSQ_ERR_ARG, std::string(fn) +
                                 ": S must be 16-byte aligned, sketches and gammas 4-byte aligned");
  const int b = beta < n_groups ? beta : n_groups;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  Workspace w;
  if ((rc = step_common(fn, s, workspace, ws_bytes, w))) return rc;
  StepTensors t{};
  t.q = q; t.l1k = l1k; t.l1k_n = l1k_n; t.l1v = l1v; t.l1v_n = l1v_n;
  t.l2k = l2k; t.l2k_n = l2k_n; t.l2v = l2v; t.l2v_n = l2v_n; t.l3 = l3; t.l3_staged = 0;
  t.k_signs = k_signs; t.v_signs = v_signs; t.cb4 = cb4; t.cb3 = cb3; t.scale = scale;
  t.summary_bias = summary_bias; t.agg = agg; t.out = out;
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = as_stream(stream);
  const QjlKeys qk0{l1_sketch, l1_gamma, l3_sketch, l3_gamma, S};
  if (s.n_groups > 0 && !route_lds_ok(s)) {  // router logits beyond LDS: the split step
    if ((rc = check_hip(launch_split_half(s, t, w, ws, true, b > 0 ? topk_idx : nullptr, st),
                        "hsq_decode_step_qjl route (split)")))
      return rc;
    return check_hip(launch_split_half(s, t, w, ws, false, nullptr, st, nullptr, &qk0),
                     "hsq_decode_step_qjl attention (split)");
  }
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx_off);
  if (s.n_groups > 0 &&
      (rc = check_hip(launch_route(s, t, w, ws, ROUTE_TOPK | ROUTE_PARTIALS, nullptr, nullptr,
                                   idx, st),
                      "hsq_decode_step_qjl route")))
    return rc;
  if ((rc = check_hip(launch_attn_qjl(s, t, w, ws, idx, qk0, st), "hsq_decode_step_qjl attention")))
    return rc;
  if (topk_idx && b > 0)
    return check_hip(hipMemcpyAsync(topk_idx, idx, sizeof(int32_t) * (size_t)B * Hkv * b,
                                    hipMemcpyDeviceToDevice, st),
                     "hsq_decode_step_qjl topk copy");
  return HSQ_OK;
}

extern "C" int hsq_decode_step_static(const float* q, int B, int Hq, int Hkv, int d,
                                      const uint8_t* l1k, const float* l1k_n, const uint8_t* l1v,
                                      const float* l1v_n, int n_l1, const uint8_t* l2k,
                                      const float* l2k_n, const uint8_t* l2v, const float* l2v_n,
                                      int n_groups, const uint8_t* l3, int group_n, int beta,
                                      int agg, const uint32_t* k_signs, const uint32_t* v_signs,
                                      const float* cb4, const float* cb3, float scale,
                                      float summary_bias, int32_t* topk_idx, float* out,
                                      void* stream) {
  const char* fn = "hsq_decode_step_static";
  int rc = check_step_shape(fn, B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  const int b = beta < n_groups ? beta : n_groups;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b};
  if (!step_limits_ok(s))
    return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": n_groups, G * n_groups or the L1/L3 "
                                     "sizes exceed the kernels' limits");
  const size_t need = plan_workspace(s).total;
  if (need > kStaticScratchBytes)
    return fail(HSQ_ERR_UNSUPPORTED,
                std::string(fn) + ": these sizes need " + std::to_string(need) +
                    " bytes of scratch; the static scratch holds " +
                    std::to_string(kStaticScratchBytes) + " (use hsq_decode_step with a workspace)");
  void* scratch = nullptr;
  if ((rc = static_scratch(&scratch))) return rc;
  return hsq_decode_step(q, B, Hq, Hkv, d, l1k, l1k_n, l1v, l1v_n, n_l1, l2k, l2k_n, l2v, l2v_n,
                         n_groups, l3, group_n, beta, agg, k_signs, v_signs, cb4, cb3, scale,
                         summary_bias, topk_idx, scratch, kStaticScratchBytes, out, stream);
}

namespace {

int gather_common(const char* fn, const uint8_t* l3_src, size_t rec_bytes, int B, int Hkv,
                  int n_groups, const int32_t* topk_idx, int beta, uint8_t* staging,
                  uint32_t* turn, uint32_t after, void* stream) {
  if (B < 1 || Hkv < 1 || n_groups < 0 || beta < 0 || beta > n_groups)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": bad sizes");
  if (rec_bytes == 0 || rec_bytes % 16)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": rec_bytes must be a positive multiple of 16");
  if (rec_bytes > (size_t(1) << 20))
    return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": rec_bytes above 1 MiB");
  if ((int64_t)B * Hkv * beta > (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": B * Hkv * beta must be < 2^32");
  if (beta == 0) return HSQ_OK;
  if (!l3_src || !topk_idx || !staging) return fail(HSQ_ERR_ARG, std::string(fn) + ": null pointer");
  return check_hip(launch_gather(l3_src, rec_bytes, B * Hkv, n_groups, topk_idx, beta, staging,
                                 turn, after, as_stream(stream)),
                   (std::string(fn) + " launch").c_str());
}

}  // namespace

extern "C" int hsq_gather_l3(const uint8_t* l3_src, size_t rec_bytes, int B, int Hkv,
                             int n_groups, const int32_t* topk_idx, int beta, uint8_t* staging,
                             void* stream) {
  return gather_common("hsq_gather_l3", l3_src, rec_bytes, B, Hkv, n_groups, topk_idx, beta,
                       staging, nullptr, 0u, stream);
}

extern "C" int hsq_gather_l3_ordered(const uint8_t* l3_src, size_t rec_bytes, int B, int Hkv,
                                     int n_groups, const int32_t* topk_idx, int beta,
                                     uint8_t* staging, uint32_t* turn, uint32_t after,
                                     void* stream) {
  if (!turn) return fail(HSQ_ERR_ARG, "hsq_gather_l3_ordered: null turn");
  if (reinterpret_cast<uintptr_t>(turn) % 4)
    return fail(HSQ_ERR_ARG, "hsq_gather_l3_ordered: turn must be 4-byte aligned");
  return gather_common("hsq_gather_l3_ordered", l3_src, rec_bytes, B, Hkv, n_groups, topk_idx,
                       beta, staging, turn, after, stream);
}

extern "C" int hsq_cache_append(const void* k_new, const void* v_new, int dtype, int B, int Hkv,
                                int d, int group_n, int n_fix, int n_recent, int64_t t,
                                int n_pending, int n_groups, int l1_cap, int ng_cap,
                                const uint32_t* k_signs, const uint32_t* v_signs,
                                const float* thr4, const float* thr3, uint8_t* l1k, float* l1k_n,
                                uint8_t* l1v, float* l1v_n, void* raw_k, void* raw_v,
                                uint8_t* l2k, float* l2k_n, uint8_t* l2v, float* l2v_n,
                                uint8_t* l3, void* stream) {
  if (B < 1 || Hkv < 1 || n_fix < 0 || n_recent < 1 || n_pending < 0 || n_groups < 0 ||
      l1_cap < 1 || ng_cap < 1)
    return fail(HSQ_ERR_ARG, "hsq_cache_append: bad sizes");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_cache_append: d must be 64 or 128");
  if (group_n != 8 && group_n != 16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_cache_append: group_n must be 8 or 16");
  if (dtype != HSQ_F32 && dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_cache_append: dtype must be HSQ_F32 or HSQ_BF16");
  if (t < n_recent) return fail(HSQ_ERR_ARG, "hsq_cache_append: t must be >= n_recent (full window)");
  if (n_pending >= group_n) return fail(HSQ_ERR_ARG, "hsq_cache_append: n_pending must be < group_n");
  if ((int64_t)n_fix + n_recent + group_n > l1_cap)
    return fail(HSQ_ERR_ARG, "hsq_cache_append: l1_cap < n_fix + n_recent + group_n");
  const bool seal = n_pending + 1 == group_n;
  if (n_groups > ng_cap || (seal && n_groups >= ng_cap))
    return fail(HSQ_ERR_ARG, "hsq_cache_append: the group capacity ng_cap is full");
  const int64_t units = (int64_t)B * Hkv;
  if (units * l1_cap >= (int64_t)UINT32_MAX || units * ng_cap >= (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_cache_append: B * Hkv * capacity must be < 2^32");
  if (!k_new || !v_new || !k_signs || !v_signs || !thr4 || !thr3 || !l1k || !l1k_n || !l1v ||
      !l1v_n || !raw_k || !raw_v || !l2k || !l2k_n || !l2v || !l2v_n || !l3)
    return fail(HSQ_ERR_ARG, "hsq_cache_append: null pointer");
  AppendJob j{k_new, v_new, dtype, (int)units, Hkv, d, group_n, n_fix, n_recent,
              (int)(t % n_recent), n_pending, l1_cap, ng_cap, n_groups, seal ? 1 : 0,
              k_signs, v_signs, thr4, thr3, l1k, l1k_n, l1v, l1v_n, raw_k, raw_v,
              l2k, l2k_n, l2v, l2v_n, l3};
  return check_hip(launch_cache_append(j, as_stream(stream)), "hsq_cache_append");
}

extern "C" int hsq_cache_decode_step(const float* q, int B, int Hq, int Hkv, int d,
                                     const uint8_t* l1k, const float* l1k_n, const uint8_t* l1v,
                                     const float* l1v_n, int n_l1, int l1_cap,
                                     const uint8_t* l2k, const float* l2k_n, const uint8_t* l2v,
                                     const float* l2v_n, int n_groups, int ng_cap,
                                     const uint8_t* l3, int group_n, int beta, int agg,
                                     const uint32_t* k_signs, const uint32_t* v_signs,
                                     const float* cb4, const float* cb3, float scale,
                                     float summary_bias, int32_t* topk_idx, void* workspace,
                                     size_t ws_bytes, float* out, void* stream) {
  const char* fn = "hsq_cache_decode_step";
  int rc = check_step_shape(fn, B, Hq, Hkv, d, n_l1, n_groups, group_n, beta);
  if (rc) return rc;
  if (l1_cap < n_l1 || ng_cap < n_groups || l1_cap < 1 || ng_cap < 1)
    return fail(HSQ_ERR_ARG, "hsq_cache_decode_step: capacities below the counts");
  if ((int64_t)B * Hkv * l1_cap >= (int64_t)UINT32_MAX ||
      (int64_t)B * Hkv * ng_cap >= (int64_t)UINT32_MAX)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_cache_decode_step: B * Hkv * capacity must be < 2^32");
  if ((rc = attn_args(fn, q, l1k, l1k_n, l1v, l1v_n, n_l1, l2k, l2k_n, l2v, l2v_n, n_groups, l3,
                      k_signs, v_signs, cb4, cb3, out)))
    return rc;
  if (agg != HSQ_AGG_MAX && agg != HSQ_AGG_MEAN) return fail(HSQ_ERR_ARG, "hsq_cache_decode_step: bad agg");
  const int b = beta < n_groups ? beta : n_groups;
  StepShape s{B, Hq, Hkv, Hq / Hkv, d, n_l1, n_groups, group_n, b, l1_cap, ng_cap};
  Workspace w;
  if ((rc = step_common(fn, s, workspace, ws_bytes, w))) return rc;
  StepTensors t{q, l1k, l1k_n, l1v, l1v_n, l2k, l2k_n, l2v, l2v_n, l3, 0,
                k_signs, v_signs, cb4, cb3, scale, summary_bias, agg, out};
  const hipStream_t st = as_stream(stream);
  if (use_split(s))
    return check_hip(launch_split_step(s, t, w, static_cast<char*>(workspace),
                                       b > 0 ? topk_idx : nullptr, st), fn);
  if (step_fused_ok(s))
    return check_hip(launch_step(s, t, b > 0 ? topk_idx : nullptr, st), fn);
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx_off);
  if ((rc = check_hip(launch_route(s, t, w, ws, ROUTE_TOPK | ROUTE_PARTIALS, nullptr, nullptr,
                                   idx, st),
                      "hsq_cache_decode_step route")))
    return rc;
  if (topk_idx && b > 0 &&
      (rc = check_hip(hipMemcpyAsync(topk_idx, idx, sizeof(int32_t) * (size_t)B * Hkv * b,
                                     hipMemcpyDeviceToDevice, st),
                      "hsq_cache_decode_step topk copy")))
    return rc;
  return check_hip(launch_attn(s, t, w, ws, idx, st), "hsq_cache_decode_step attend");
}

extern "C" int hsq_encode_qjl(const void* x, int x_dtype, int64_t n_vec, int d, int bits,
                              const uint32_t* signs, const float* thresholds,
                              const float* centroids, const float* S, uint8_t* codes,
                              float* norms, uint8_t* sketch, float* gamma, void* stream) {
  if (n_vec < 0) return fail(HSQ_ERR_ARG, "hsq_encode_qjl: n_vec must be >= 0");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode_qjl: d must be 64 or 128");
  if (!supported_bits(bits)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode_qjl: bits must be 3 or 4");
  if (x_dtype != HSQ_F32 && x_dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_encode_qjl: dtype must be HSQ_F32 or HSQ_BF16");
  if (n_vec == 0) return HSQ_OK;
  if (!x || !signs || !thresholds || !centroids || !S || !codes || !norms || !sketch || !gamma)
    return fail(HSQ_ERR_ARG, "hsq_encode_qjl: null pointer");
  QjlJob j{x, x_dtype, n_vec, d, bits, signs, thresholds, centroids, S, codes, norms, sketch,
           gamma};
  return check_hip(launch_qjl_encode(j, as_stream(stream)), "hsq_encode_qjl");
}

extern "C" int hsq_build_sketches(const void* k, int dtype, int B, int Hkv, int T, int d,
                                  const int32_t* l1_pos, int n1, const int32_t* group_pos,
                                  int n_groups, int group_n, const uint32_t* k_signs,
                                  const float* thr4, const float* cb4, const float* S,
                                  uint8_t* l1_sketch, float* l1_gamma, uint8_t* l3_sketch,
                                  float* l3_gamma, void* stream) {
  const char* fn = "hsq_build_sketches";
  if (B < 1 || Hkv < 1 || T < 1 || n1 < 0 || n_groups < 0 || group_n < 1)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": bad sizes");
  if ((int64_t)n1 + (int64_t)n_groups * group_n > T)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": n1 + n_groups * group_n exceeds T");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": d must be 64 or 128");
  if (dtype != HSQ_F32 && dtype != HSQ_BF16)
    return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": dtype must be HSQ_F32 or HSQ_BF16");
  if ((int64_t)B * Hkv * T >= (int64_t(1) << 32))
    return fail(HSQ_ERR_UNSUPPORTED, std::string(fn) + ": B * Hkv * T must be below 2^32");
  if (!k || !k_signs || !thr4 || !cb4 || !S)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null pointer");
  if (n1 > 0 && (!l1_pos || !l1_sketch || !l1_gamma))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null L1 pointer");
  if (n_groups > 0 && (!group_pos || !l3_sketch || !l3_gamma))
    return fail(HSQ_ERR_ARG, std::string(fn) + ": null archive pointer");
  if (reinterpret_cast<uintptr_t>(l1_sketch) % 2 || reinterpret_cast<uintptr_t>(l3_sketch) % 2)
    return fail(HSQ_ERR_ARG, std::string(fn) + ": sketch arrays must be 2-byte aligned");
  const hipStream_t st = as_stream(stream);
  for (int h = 0; h < Hkv; ++h) {
    for (int tier = 0; tier < 2; ++tier) {
      const int64_t per_seq = tier == 0 ? n1 : (int64_t)n_groups * group_n;
      if (per_seq == 0) continue;
      QjlJob j{};
      j.x = k; j.dtype = dtype; j.n_vec = (int64_t)B * per_seq; j.d = d; j.bits = 4;
      j.signs = k_signs + (size_t)h * (d / 32); j.thr = thr4; j.centroids = cb4;
      j.S = S + (size_t)h * d * d;
      j.sketch = tier == 0 ? l1_sketch : l3_sketch;
      j.gamma = tier == 0 ? l1_gamma : l3_gamma;
      j.pos = tier == 0 ? l1_pos : group_pos;
      j.per_seq = per_seq; j.x_seq = (int64_t)Hkv * T; j.x_base = (int64_t)h * T;
      j.out_seq = (int64_t)Hkv * per_seq; j.out_base = (int64_t)h * per_seq;
      const int rc = check_hip(launch_qjl_encode(j, st), "hsq_build_sketches");
      if (rc) return rc;
    }
  }
  return HSQ_OK;
}

extern "C" int hsq_qjl_logits(const float* q, int n_q, int d, int bits, const uint8_t* codes,
                              const float* norms, const uint8_t* sketch, const float* gamma,
                              int64_t n_keys, const uint32_t* signs, const float* centroids,
                              const float* S, float scale, float* out, void* stream) {
  if (n_q < 1 || n_q > 8 || n_keys < 0)
    return fail(HSQ_ERR_ARG, "hsq_qjl_logits: n_q must be in 1..8, n_keys >= 0");
  if (!supported_d(d)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_qjl_logits: d must be 64 or 128");
  if (!supported_bits(bits)) return fail(HSQ_ERR_UNSUPPORTED, "hsq_qjl_logits: bits must be 3 or 4");
  if (n_keys >= (int64_t)UINT32_MAX * 256)
    return fail(HSQ_ERR_UNSUPPORTED, "hsq_qjl_logits: too many keys");
  if (n_keys == 0) return HSQ_OK;
  if (!q || !codes || !norms || !sketch || !gamma || !signs || !centroids || !S || !out)
    return fail(HSQ_ERR_ARG, "hsq_qjl_logits: null pointer");
  QjlLogitsJob j{q, n_q, d, bits, codes, norms, sketch, gamma, n_keys, signs, centroids, S, scale,
                 out};
  return check_hip(launch_qjl_logits(j, as_stream(stream)), "hsq_qjl_logits");
}
