// Internal interface between the C-ABI front end (sdpa_api.hip) and the
// kernel files. Not installed; not part of the public header.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace sdpa {

// Element strides (b, h, s) of one logical (b, h, s, d) tensor; d stride is 1.
struct Strides3 {
  int64_t b, h, s;
};

// Score modifiers (additive bias tensor, ALiBi), added to the scaled scores
// before the mask: S += bias[b][h][i][j] - slopes[h] * |i + off - j|.
struct ScoreMod {
  const float* slopes;  // device fp32 [h_q], or null
  const void* bias;     // device bias (fp32, or 16-bit of the io type), or null
  int bias_f32;         // 1: fp32 bias, 0: 16-bit
  int64_t bb, bh, bs;   // element strides of the bias in (b, h, s_q); s_kv stride 1; 0 broadcasts
  // Dropout of the attention weights: element (i, j) of query-head slot
  // b * h_q + h is kept iff byte (j % 4) of word (i % 4) of
  // Philox4x32-10(counter (j / 4, i / 4, slot, offset), key (seed_lo, seed_hi))
  // is below drop_k8; kept weights are scaled by drop_scale = 256 / drop_k8.
  int drop_k8;          // 256: no dropout
  float drop_scale;
  uint32_t seed_lo, seed_hi, offset;
};

// Whether any modifier is active (the kernels take their MOD variant).
inline bool has_mod(const ScoreMod& m) { return m.slopes != nullptr || m.bias != nullptr || m.drop_k8 < 256; }

// Kernel variants by score modifier: none; ALiBi slopes only (no loads beyond
// one slope per head, no random numbers); dropout, with or without ALiBi (no
// bias loads); the general path (a bias tensor, with ALiBi and dropout).
constexpr int kModNone = 0, kModAlibi = 1, kModDrop = 2, kModAll = 3;
inline int mod_level(const ScoreMod& m) {
  if (!has_mod(m)) return kModNone;
  if (m.bias != nullptr) return kModAll;
  return m.drop_k8 < 256 ? kModDrop : kModAlibi;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  Strides3 qs, ks, vs, os;
  int b, h_q, h_kv, s_q, s_kv, d;
  int causal;
  int bottom_right;        // causal diagonal aligned to the end of the key range
  const int32_t* seq_q;    // device [b] valid query rows, or null (= s_q)
  const int32_t* seq_kv;   // device [b] valid keys, or null (= s_kv)
  ScoreMod mod;            // bias / ALiBi (both null: none)
  float scale;  // attn_scale (already multiplied by the fp8 q/k descales for fp8)
  // fp8 only
  float descale_v, scale_p, descale_p;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  Strides3 qs, ks, vs, os, dos, dqs, dks, dvs;
  int b, h_q, h_kv, s_q, s_kv, d;
  int causal;
  int bottom_right;
  const int32_t* seq_q;
  const int32_t* seq_kv;
  ScoreMod mod;
  float scale;        // multiplies Q K^T inside the softmax
  float dq_scale;     // dQ = dq_scale * dS K      (scale for real-valued inputs)
  float dk_scale;     // dK = dk_scale * dS^T Q    (scale)
  float dv_scale;     // dV = dv_scale * P^T dO    (1)
  float delta_scale;  // D_i = delta_scale * sum_d dO_id * O_id (1)
  float* delta;  // workspace: fp32 [b][h_q][s_q], D_i = sum_d dO_id * O_id
  // fp8 backward only (codes in, the 16-bit path ignores these)
  struct {
    float dp_scale;   // dP = dp_scale * (dO codes . V codes)
    float scale_p;    // P is quantised to e4m3 as P * scale_p
    float scale_ds;   // dS is quantised as dS * scale_ds (saturating)
    float* amax_ds;   // optional: max-combined with max |dS| (bit pattern, >= 0)
    int do_e5m2;      // dO codes are e5m2 (else e4m3)
    int ds_e5m2;      // dS is quantised to e5m2 (else e4m3)
  } f8;
};

// Split-KV forward (few query rows, many keys): partial results of each key
// split, merged by a second kernel.
struct DecodeArgs {
  int n_split;      // key splits per (batch, KV head, row block)
  int split_keys;   // keys per split (multiple of the key tile)
  int n_rb;         // 32-row blocks per KV group (rows = (h_q / h_kv) * s_q)
  float* part_o;    // [n_split][b][h_q][s_q][d] fp32 O / l per split (n_split > 1)
  float* part_lse;  // [n_split][b][h_q][s_q] natural-log LSE per split, -inf if empty
};

struct DecodePlan {
  bool use;         // the split-KV path applies to this shape
  int n_split, split_keys, n_rb;
  size_t ws_bytes;  // workspace it needs (0 when n_split == 1)
};

// Caller events recorded at kernel boundaries (timing hook); n = 0 disables.
struct TimingEvents {
  hipEvent_t ev[8];
  int n;
};

enum class Io { F32, F16, BF16, FP8 };

// Kernel launchers; each returns hipGetLastError() after enqueueing.
hipError_t launch_fwd_mfma(const FwdArgs& a, Io io, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream);
DecodePlan plan_decode(int b, int h_q, int h_kv, int s_q, int s_kv, int d, Io io);
hipError_t launch_fwd_decode(const FwdArgs& a, const DecodePlan& p, void* workspace, Io io, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, Io io, hipStream_t stream, const TimingEvents& te);
// fp8 backward (codes in a.q, a.k, a.v, a.dout; bf16 o, dq, dk, dv); d 64 or 128.
hipError_t launch_bwd_fp8(const BwdArgs& a, hipStream_t stream, const TimingEvents& te);
hipError_t launch_zero_dkdv(const BwdArgs& a, Io io, hipStream_t stream);
// Query-head split of the dK/dV kernels (1: none) and, when it is > 1, their
// fp32 partials in the workspace after D, and the kernel that sums them in
// split order into bf16 dK, dV.
int bwd_split_count(int b, int h_q, int h_kv, int s_kv, int keys_per_wg);
float* bwd_partials(const BwdArgs& a);
hipError_t launch_bwd_reduce(const BwdArgs& a, int n_split, const float* part, hipStream_t stream);

// Matrix-core rate probe (bf16 32x32x16 or fp8 32x32x64 MFMAs); stamps get
// 4 uint64 per workgroup: shader cycles and real time at loop start and end.
hipError_t launch_mfma_probe(bool fp8, int blocks, int iters, uint64_t* stamps, hipStream_t stream);

// Workspace bytes the backward needs (see sdpa_bwd_workspace_size).
size_t bwd_workspace_bytes(int b, int h_q, int h_kv, int s_q, int s_kv, int d);

}  // namespace sdpa
