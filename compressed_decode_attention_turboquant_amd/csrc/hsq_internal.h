// Internal declarations shared by the libhsq translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "hsq.h"

namespace hsq {

// ---- error reporting (api.cpp) -------------------------------------------
int fail(int code, const std::string& msg);
int check_hip(hipError_t e, const char* what);

// ---- encode / decode (codec.hip) -----------------------------------------
struct EncodeJob {
  const void* x;
  int dtype;          // HSQ_F32 / HSQ_BF16
  int64_t n_vec;
  int d;
  int bits;
  int group_n;        // rows averaged per output vector
  // row mapping: row_idx (direct) | pos (tier build) | contiguous
  const int64_t* row_idx;
  const int32_t* pos;
  int64_t vecs_per_unit;
  int64_t rows_per_unit;
  int64_t units_per_seq;
  int64_t pos_per_seq;
  // rotation: mask (i / vecs_per_rot) % n_rot
  const uint32_t* signs;
  int64_t vecs_per_rot;
  int64_t n_rot;
  const float* thr;
  // output: vector i -> record i / vecs_per_rec, slot i % vecs_per_rec
  uint8_t* codes;
  int64_t code_rec_bytes;
  float* norms;
  int64_t norm_rec_floats;
  int64_t vecs_per_rec;
};
hipError_t launch_encode(const EncodeJob& j, hipStream_t s);

struct DecodeJob {
  const uint8_t* codes;
  const float* norms;
  int64_t n_vec;
  int d;
  int bits;
  const uint32_t* signs;
  int64_t vecs_per_rot;
  int64_t n_rot;
  const float* centroids;
  void* out;
  int out_dtype;
  // RoPE at fetch: when pos is set, row i is rotated to position pos[i]
  // with the rotary base rope_base after dequantisation
  const int32_t* pos;
  double rope_base;
};
hipError_t launch_decode(const DecodeJob& j, hipStream_t s);

// Fetched keys of a pre-RoPE archive (codec.hip): for every selection slot s
// of every unit u and token t of the group, the 4-bit key of the record in
// the rotated domain (unit norm), taken back to the model's domain and
// rotated to the token's position: fp16 out[u][s][t][d], the rows the attend
// kernel multiplies against the unrotated query in place of the table
// lookups.
struct RopeKeysJob {
  const uint8_t* l3;        // archive records, N * (d + 8) bytes each
  int64_t unit_recs;        // records between consecutive units (n_groups or a capacity)
  const int32_t* idx;       // [units][beta] selected group per slot
  const int32_t* group_pos; // [B][pos_per_seq] token positions, group-major
  int64_t pos_per_seq;
  int units, Hkv, d, n_groups, group_n, beta;
  const uint32_t* k_signs;  // [Hkv][d/32]
  const float* cb4;         // 16 centroids
  double rope_base;
  uint16_t* out;            // fp16 bits [units][beta][group_n][d]
  int staged;               // records gathered by slot: [units][beta] (unit_recs unused)
};
hipError_t launch_rope_keys(const RopeKeysJob& j, hipStream_t s);

// ---- decode step (route.hip / attn.hip) ------------------------------------
struct StepShape {
  int B, Hq, Hkv, G, d;
  int n_l1, n_groups, group_n, beta;  // beta already clamped to [0, n_groups]
  // rows between consecutive units of the L1 arrays and groups between those
  // of the L2 / L3 arrays (capacities of a decode-time cache); 0 = n_l1 /
  // n_groups (dense tiers)
  int l1_stride, ng_stride;
};

struct StepTensors {
  const float* q;
  const uint8_t* l1k; const float* l1k_n; const uint8_t* l1v; const float* l1v_n;
  const uint8_t* l2k; const float* l2k_n; const uint8_t* l2v; const float* l2v_n;
  const uint8_t* l3; int l3_staged;
  const uint32_t* k_signs; const uint32_t* v_signs;
  const float* cb4; const float* cb3;
  float scale, summary_bias;
  int agg;
  float* out;
};

// Workspace layout (all offsets 256-byte aligned).
struct Workspace {
  size_t idx_off;      // int32 [B*Hkv][beta]   selection
  size_t part_off;     // fp32  [B*Hkv][G][d+2] summary-attention partial (m, l, O)
  // split step only (split_shape): per-head logits, router keys, largest key
  // norm per score chunk, selection bitmap, partials of the attend chunks
  size_t lgt_off, keys_off, rn_off, bits_off, parts_off;
  size_t total;
};
Workspace plan_workspace(const StepShape& s);
// shapes the step kernels can address (group count, 32-bit buffer offsets)
int step_limits_ok(const StepShape& s);
// shapes whose router logits fit in LDS (one-launch step, two-launch route)
int route_lds_ok(const StepShape& s);
// shapes the split kernels serve (and whose workspace holds their buffers):
// few units, or router logits beyond LDS
int split_shape(const StepShape& s);
// shapes hsq_decode_step runs as the split step: split shapes the one-launch
// step cannot take (more than 2048 groups, or LDS)
int use_split(const StepShape& s);
hipError_t launch_split_step(const StepShape& s, const StepTensors& t, const Workspace& w,
                             char* ws, int32_t* idx_out, hipStream_t st);
// The split step in two calls (split_shape shapes): first = scores, selection
// (idx_out optional) and the summary-value chunks, from t's router inputs;
// else the token chunks (L1 and the fetched records; staged ones by slot)
// and the merge, from t's attend inputs.  Same shape and workspace in both.
// The second half may run the pre-RoPE tiles (kdense: the fetched keys'
// fp16 rows) or the TQ-QKV tiles (qk), as launch_attn_prerope / _qjl do.
struct QjlKeys;
hipError_t launch_split_half(const StepShape& s, const StepTensors& t, const Workspace& w,
                             char* ws, bool first, int32_t* idx_out, hipStream_t st,
                             const uint16_t* kdense = nullptr, const QjlKeys* qk = nullptr);

// mode bits for the summary kernel
enum { ROUTE_TOPK = 1, ROUTE_PARTIALS = 2 };

hipError_t launch_route(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                        int mode, const int32_t* given_idx, float* scores_out,
                        int32_t* idx_out, hipStream_t st);
hipError_t launch_attn(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                       const int32_t* idx, hipStream_t st);
// launch_attn over a pre-RoPE archive: the fetched tiles multiply the fp16
// model-domain key rows kdense [units][beta][group_n][d] (launch_rope_keys)
// against the unrotated query instead of the records' key codes against the
// rotated one (kdense may be null when beta == 0)
hipError_t launch_attn_prerope(const StepShape& s, const StepTensors& t, const Workspace& w,
                               char* ws, const int32_t* idx, const uint16_t* kdense,
                               hipStream_t st);
// launch_attn over TQ-QKV token keys (dense tiers, device archive): every L1
// and fetched token's logit gains its QJL residual estimate from the sketch
// arrays and the sketch matrices S [Hkv][d][d]
struct QjlKeys {
  const uint8_t* l1_sk; const float* l1_gam;  // [units][n1][d/8], [units][n1]
  const uint8_t* l3_sk; const float* l3_gam;  // [units][ng][N][d/8], [units][ng][N]
  const float* S;
};
hipError_t launch_attn_qjl(const StepShape& s, const StepTensors& t, const Workspace& w, char* ws,
                           const int32_t* idx, const QjlKeys& qk, hipStream_t st);
// The whole step in one launch (route + attend per work-group); only for
// shapes where step_fused_ok holds.  idx_out (optional): [units][beta].
int step_fused_ok(const StepShape& s);
hipError_t launch_step(const StepShape& s, const StepTensors& t, int32_t* idx_out,
                       hipStream_t st);
// turn == nullptr: plain gather; else wait (bounded) for *turn >= after,
// then add the records moved to *turn
hipError_t launch_gather(const uint8_t* src, size_t rec_bytes, int units, int n_groups,
                         const int32_t* idx, int beta, uint8_t* dst, uint32_t* turn,
                         uint32_t after, hipStream_t st);

// ---- decode-time tier maintenance (cache.hip) -------------------------------
// One token appended per unit; layouts as in include/hsq.h ("Cache layout").
struct AppendJob {
  const void* k_new; const void* v_new; int dtype;  // [units][d] raw
  int units, Hkv, d, group_n, n_fix, n_recent, slot, pending, l1_cap, ng_cap, ng, seal;
  const uint32_t* k_signs; const uint32_t* v_signs;
  const float* thr4; const float* thr3;
  uint8_t* l1k; float* l1k_n; uint8_t* l1v; float* l1v_n;
  void* raw_k; void* raw_v;                          // [units][W + N][d]
  uint8_t* l2k; float* l2k_n; uint8_t* l2v; float* l2v_n;
  uint8_t* l3;
};
hipError_t launch_cache_append(const AppendJob& j, hipStream_t s);

// ---- TQ-QKV key path (qjl.hip) -----------------------------------------------
// Keys of one rotation (one sign mask, one sketch matrix S [d][d] fp32).
struct QjlJob {
  const void* x; int dtype; int64_t n_vec; int d, bits;
  const uint32_t* signs; const float* thr; const float* centroids; const float* S;
  uint8_t* codes; float* norms; uint8_t* sketch; float* gamma;
  // gathered rows (tier build), when pos is set: vector i = (s, t) with
  // s = i / per_seq, t = i % per_seq reads row x_base + s * x_seq + pos[i]
  // of x and writes its sketch and gamma at out_base + s * out_seq + t;
  // codes and norms may be null (not written)
  const int32_t* pos; int64_t per_seq, x_seq, x_base, out_seq, out_base;
};
hipError_t launch_qjl_encode(const QjlJob& j, hipStream_t s);
struct QjlLogitsJob {
  const float* q; int n_q, d, bits;
  const uint8_t* codes; const float* norms; const uint8_t* sketch; const float* gamma;
  int64_t n_keys;
  const uint32_t* signs; const float* centroids; const float* S; float scale;
  float* out;
};
hipError_t launch_qjl_logits(const QjlLogitsJob& j, hipStream_t s);

// ---- device scratch of the entry points that allocate nothing (scratch.hip) --
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
// Address of this device's scratch array (looked up on the first call on
// each device, with that device current).
int static_scratch(void** out);

// ---- host-side method pieces (host.cpp) -------------------------------------
int codebook(int d, int bits, float* centroids, float* thresholds);

}  // namespace hsq
