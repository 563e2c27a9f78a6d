// FP32 forward on the fp32 matrix cores (v_mfma_f32_32x32x2_f32): fused
// attention with fp32 inputs and outputs (JAX attention codelab, step 1
// formula and step 7 causal mask; cuDNN 9 blog, "SDPA as a cuDNN graph",
// Figure 4; the padding mask, bias and ALiBi of the node's options).
//
// Layout (the transposed-score form of the 16-bit forward):
//  * S^T = K Q^T, 32 keys x 32 query rows per wave and tile. The 32x32x2
//    MFMA contracts one index per lane half, so lane half h walks d in
//    [D/2 h, D/2 h + D/2): the lane's Q values (B operand, registers, scaled
//    by attn_scale * log2 e) and K values (A operand, 16-byte LDS reads of a
//    row-padded tile) are both contiguous.
//  * Accumulator register r of lane (query j, half h) is key 8 (r/4) + 4 h +
//    r % 4. O^T += V^T P^T takes register u of the weights as the B operand of
//    step u directly (step u pairs the keys of register u in the two halves),
//    so the weights never move; the matching V^T values are four consecutive
//    keys per 16-byte read of a transposed, row-padded V tile.
//  * Exact online softmax (row max per tile, rescale on every increase).
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

constexpr int kNW32 = 4;   // waves per workgroup, 32 query rows each
constexpr int kBN32 = 32;  // keys per tile

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL, bool MOD>
__global__ __launch_bounds__(64 * kNW32) void fwd_f32_mfma_kernel(FwdArgs a, int n_qblk) {
  constexpr int NT = 64 * kNW32;
  constexpr int BM = 32 * kNW32;    // query rows per workgroup
  constexpr int HD = D / 2;         // d values one lane half contracts
  constexpr int NDB = D / 32;       // 32-wide output blocks over d
  // Row pitches (floats) 16 bytes past a multiple of 64 bytes: the 16-byte
  // reads of 16 lanes at one column of 16 consecutive rows hit distinct bank
  // groups.
  constexpr int KSTR = D + 4;       // K tile
  constexpr int VSTR = kBN32 + 4;   // transposed V tile
  __shared__ __attribute__((aligned(16))) float Ks[kBN32 * KSTR];
  __shared__ __attribute__((aligned(16))) float Vt[D * VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int bh_total = a.b * a.h_q;
  const int bh = blockIdx.x % bh_total;
  const int qb = n_qblk - 1 - blockIdx.x / bh_total;  // longest causal blocks first
  const int bi = bh / a.h_q, hq = bh % a.h_q;
  const int g = hq / (a.h_q / a.h_kv);
  const int qblk0 = qb * BM;
  const int q0 = qblk0 + 32 * wave;
  const int my_q = q0 + j;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);
  const float* qp = (const float*)a.q + bi * a.qs.b + hq * a.qs.h;
  const float* kp = (const float*)a.k + bi * a.ks.b + g * a.ks.h;
  const float* vp = (const float*)a.v + bi * a.vs.b + g * a.vs.h;
  const float sl2 = a.scale * kLog2e;

  // Q row my_q, d = HD h + t, scaled into log2 units (B operand of S^T).
  float qf[HD];
#pragma unroll
  for (int t4 = 0; t4 < HD / 4; ++t4) {
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
    if (my_q < L.lq) x = *(const f32x4*)(qp + (int64_t)my_q * a.qs.s + HD * h + 4 * t4);
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[4 * t4 + e] = x[e] * sl2;
  }
  const float slope = (MOD && a.mod.slopes != nullptr) ? a.mod.slopes[hq] : 0.f;
  const float* bias_row = (MOD && a.mod.bias != nullptr && my_q < a.s_q)
                              ? (const float*)a.mod.bias + bi * a.mod.bb + hq * a.mod.bh + (int64_t)my_q * a.mod.bs
                              : nullptr;

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane half's keys
  const int kv_end = qblk0 >= L.lq ? 0 : CAUSAL ? max(0, min(L.lk, min(qblk0 + BM, L.lq) + L.off)) : L.lk;
  for (int k0 = 0; k0 < kv_end; k0 += kBN32) {
    __syncthreads();  // every wave is done with the previous tile
    for (int c = tid; c < kBN32 * D / 4; c += NT) {
      const int r = c / (D / 4), d4 = 4 * (c % (D / 4));
      f32x4 kx = f32x4{0.f, 0.f, 0.f, 0.f}, vx = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k0 + r < L.lk) {  // keys at or past lk are zero (and masked)
        kx = *(const f32x4*)(kp + (int64_t)(k0 + r) * a.ks.s + d4);
        vx = *(const f32x4*)(vp + (int64_t)(k0 + r) * a.vs.s + d4);
      }
      *(f32x4*)(&Ks[r * KSTR + d4]) = kx;
#pragma unroll
      for (int e = 0; e < 4; ++e) Vt[(d4 + e) * VSTR + r] = vx[e];
    }
    __syncthreads();  // the tile is in LDS
    if (CAUSAL && k0 > q0 + 31 + L.off) continue;  // every key of the tile is above this wave's rows

    f32x16 s = f32x16{};
#pragma unroll
    for (int t4 = 0; t4 < HD / 4; ++t4) {
      const f32x4 kv = *(const f32x4*)(&Ks[j * KSTR + HD * h + 4 * t4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma_f32(kv[e], qf[4 * t4 + e], s);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + acc_row(r, h);
      float x = s[r];
      if (MOD) {  // + (bias - slope * |i + off - j|) * log2 e
        const float bv = (bias_row != nullptr && key < a.s_kv) ? bias_row[key] : 0.f;
        x = fmaf(bv - slope * fabsf((float)(my_q + L.off - key)), kLog2e, x);
      }
      if (key >= L.lk || (CAUSAL && key > my_q + L.off)) x = -INFINITY;
      s[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = wave_max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    // m stays -inf while every score of the row is -inf: P = 0, nothing to rescale.
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(s[r] - msub);
      l_run += s[r];
    }
    // O^T += V^T P^T: step u pairs keys acc_row(u, 0) and acc_row(u, 1).
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 va = *(const f32x4*)(&Vt[(32 * db + j) * VSTR + 8 * q4 + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db] = mfma_f32(va[e], s[4 * q4 + e], oacc[db]);
      }
  }
  const float l_tot = wave_sum_halves(l_run);
  if (my_q < a.s_q) {
    // Rows past lq, and rows that see no key: O = 0, LSE = -inf.
    const bool live = my_q < L.lq && l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    float* op = (float*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)my_q * a.os.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(f32x4*)(op + 32 * db + 8 * rq + 4 * h) =
            f32x4{oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv, oacc[db][4 * rq + 2] * inv,
                  oacc[db][4 * rq + 3] * inv};
    if (a.lse != nullptr && h == 0)
      a.lse[((int64_t)bi * a.h_q + hq) * a.s_q + my_q] = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_f32_d(const FwdArgs& a, hipStream_t stream) {
  const int n_qblk = (a.s_q + 32 * kNW32 - 1) / (32 * kNW32);
  const dim3 grid(n_qblk * a.b * a.h_q), block(64 * kNW32);
  const bool mod = has_mod(a.mod);
  if (a.causal) {
    if (mod)
      hipLaunchKernelGGL((fwd_f32_mfma_kernel<D, true, true>), grid, block, 0, stream, a, n_qblk);
    else
      hipLaunchKernelGGL((fwd_f32_mfma_kernel<D, true, false>), grid, block, 0, stream, a, n_qblk);
  } else {
    if (mod)
      hipLaunchKernelGGL((fwd_f32_mfma_kernel<D, false, true>), grid, block, 0, stream, a, n_qblk);
    else
      hipLaunchKernelGGL((fwd_f32_mfma_kernel<D, false, false>), grid, block, 0, stream, a, n_qblk);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_f32_d<64>(a, stream) : launch_f32_d<128>(a, stream);
}

}  // namespace sdpa
