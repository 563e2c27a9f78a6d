// Backward kernels: exact gradient of the fused attention forward.
//
// The pages show only that a forward + backward SDPA exists (cuDNN 9 blog,
// "SDPA performance", Figure 2, and in "SDPA as a cuDNN graph": the backward
// attention graph has similar flexibility); the backward here is the exact
// chain-rule gradient, recomputing the softmax weights from the forward's
// logsumexp (its "stats" output):
//   P = exp(scale * Q K^T - LSE)  (masked entries 0)
//   D_i = sum_d dO_id O_id
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q
// with dK/dV summed over the query heads that share a KV head (JAX attention
// codelab, step 9: KV heads shared by a group of query heads).
//
// Kernels (all atomic-free and deterministic):
//  1. delta:  D = rowsum(dO * O) in fp32 (memory-bound).
//  2. dK/dV:  KV-stationary. A workgroup owns 128 keys (32 per wave, held in
//     registers); it loops over the query heads of its group and over 32-row
//     query tiles, which are staged in LDS both row-major and transposed.
//     Each lane owns one key column of S = Q K^T, so P and dS are directly the
//     B operands of dV^T += dO^T P and dK^T += Q^T dS.
//     When a GQA/MQA group would leave the GPU underfilled, the group's query
//     heads are split over several workgroups that write fp32 partials.
//  3. reduce: sums the partials of the splits in a fixed order.
//  4. dQ:     Q-stationary, laid out like the forward: each lane owns one
//     query column of S^T = K Q^T; dQ^T += K^T dS^T with K^T read from a
//     transposed LDS copy of the K tile.
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

constexpr int kKvBlock = 128;  // keys per dK/dV workgroup (4 waves x 32)
constexpr int kQTile = 32;     // query rows per dK/dV inner step
constexpr int kQBlock = 128;   // query rows per dQ workgroup (4 waves x 32)
constexpr int kKTile = 64;     // keys per dQ inner step

// D_i = sum_d dO_id * O_id (fp32); a group of d/8 lanes per row, 16-byte loads.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per block
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  const int64_t total = (int64_t)a.b * a.h_q * a.s_q;
  float acc = 0.f;
  if (r < total) {
    const int i = (int)(r % a.s_q);
    const int64_t bh = r / a.s_q;
    const int hq = (int)(bh % a.h_q), bi = (int)(bh / a.h_q);
    const uint16_t* op = (const uint16_t*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)i * a.os.s + part * 8;
    const uint16_t* dp = (const uint16_t*)a.dout + bi * a.dos.b + hq * a.dos.h + (int64_t)i * a.dos.s + part * 8;
    const u32x4 ov = *(const u32x4*)op, dv = *(const u32x4*)dp;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(to_f32<T>((uint16_t)(ov[w] & 0xffff)), to_f32<T>((uint16_t)(dv[w] & 0xffff)), acc);
      acc = fmaf(to_f32<T>((uint16_t)(ov[w] >> 16)), to_f32<T>((uint16_t)(dv[w] >> 16)), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < total && part == 0) a.delta[r] = acc;
}

// Writes zeros to dK and dV (problems with no query rows).
__global__ __launch_bounds__(256) void zero_dkdv_kernel(BwdArgs a) {
  const int64_t chunks_per_row = a.d / 8;
  const int64_t total = (int64_t)a.b * a.h_kv * a.s_kv * chunks_per_row;
  for (int64_t c = blockIdx.x * 256LL + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
    const int64_t row = c / chunks_per_row;
    const int part = (int)(c % chunks_per_row);
    const int j = (int)(row % a.s_kv);
    const int64_t bh = row / a.s_kv;
    const int g = (int)(bh % a.h_kv), bi = (int)(bh / a.h_kv);
    *(u32x4*)((uint16_t*)a.dk + bi * a.dks.b + g * a.dks.h + (int64_t)j * a.dks.s + part * 8) = u32x4{0, 0, 0, 0};
    *(u32x4*)((uint16_t*)a.dv + bi * a.dvs.b + g * a.dvs.h + (int64_t)j * a.dvs.s + part * 8) = u32x4{0, 0, 0, 0};
  }
}

// Stages rows [row0, row0 + R) x D of a 16-bit tensor (rows >= n_rows are
// zero) into LDS twice: row-major (stride D + 8) and transposed (stride R + 4),
// via 4x4 blocks loaded as 8-byte row pieces.
template <int R, int D>
__device__ __forceinline__ void stage_both(const uint16_t* src, int64_t row_stride, int row0, int n_rows,
                                           uint16_t* rm, uint16_t* tr, int tid) {
  constexpr int DG = D / 4;
  constexpr int RS = D + 8, TS = R + 4;
#pragma unroll
  for (int c = tid; c < (R / 4) * DG; c += 256) {
    const int dg = c % DG, rg = c / DG;
    u32x2 rows[4], cols[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * rg + r;
      rows[r] = u32x2{0, 0};
      if (row < n_rows) rows[r] = *(const u32x2*)(src + (int64_t)row * row_stride + 4 * dg);
      *(u32x2*)(&rm[(4 * rg + r) * RS + 4 * dg]) = rows[r];
    }
    transpose4x4_b16(rows, cols);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) *(u32x2*)(&tr[(4 * dg + c2) * TS + 4 * rg]) = cols[c2];
  }
}

// Stages rows [row0, row0 + R) x D row-major (stride D + 8), zero beyond n_rows.
template <int R, int D>
__device__ __forceinline__ void stage_rm(const uint16_t* src, int64_t row_stride, int row0, int n_rows,
                                         uint16_t* rm, int tid) {
  constexpr int CH = D / 8;
  constexpr int RS = D + 8;
#pragma unroll
  for (int c = tid; c < R * CH; c += 256) {
    const int r = c / CH, cc = c - (c / CH) * CH;
    u32x4 val = u32x4{0, 0, 0, 0};
    if (row0 + r < n_rows) val = *(const u32x4*)(src + (int64_t)(row0 + r) * row_stride + cc * 8);
    *(u32x4*)(&rm[r * RS + cc * 8]) = val;
  }
}

// Stages rows [row0, row0 + R) x D transposed (stride R + 4), zero beyond n_rows.
template <int R, int D>
__device__ __forceinline__ void stage_tr(const uint16_t* src, int64_t row_stride, int row0, int n_rows,
                                         uint16_t* tr, int tid) {
  constexpr int DG = D / 4;
  constexpr int TS = R + 4;
#pragma unroll
  for (int c = tid; c < (R / 4) * DG; c += 256) {
    const int dg = c % DG, rg = c / DG;
    u32x2 rows[4], cols[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * rg + r;
      rows[r] = u32x2{0, 0};
      if (row < n_rows) rows[r] = *(const u32x2*)(src + (int64_t)row * row_stride + 4 * dg);
    }
    transpose4x4_b16(rows, cols);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) *(u32x2*)(&tr[(4 * dg + c2) * TS + 4 * rg]) = cols[c2];
  }
}

// A operand taken from a transposed LDS tile (row = feature index f, stride TS):
// lane half h element m stands for row key_of(t, h, m) of the original tile.
template <typename V8>
__device__ __forceinline__ V8 read_tr_operand(const uint16_t* tr, int TS, int f, int t, int h) {
  const uint16_t* p = tr + f * TS + 16 * t + 4 * h;
  const u32x2 lo = *(const u32x2*)(p);
  const u32x2 hi = *(const u32x2*)(p + 8);
  return __builtin_bit_cast(V8, u32x4{lo.x, lo.y, hi.x, hi.y});
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a, int n_kblk, int n_split, float* part) {
  typedef typename T::vec8 V8;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int RS = D + 8, TS = kQTile + 4;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kQTile * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Ds_[kQTile * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Dt[D * TS];
  __shared__ __attribute__((aligned(16))) float lse2s[kQTile];
  __shared__ __attribute__((aligned(16))) float dels[kQTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int n_slots = a.b * a.h_kv * n_split;
  // Linear id -> (key block, slot); causal: key block 0 (the most query tiles) first.
  const int kb = blockIdx.x / n_slots;
  int slot = blockIdx.x - kb * n_slots;
  if ((n_slots & 7) == 0) {
    const int per = n_slots >> 3;
    slot = (slot & 7) * per + (slot >> 3);
  }
  const int sp = slot % n_split;
  const int bg = slot / n_split;
  const int g = bg % a.h_kv, bi = bg / a.h_kv;
  const int G = a.h_q / a.h_kv, Gs = G / n_split;
  (void)n_kblk;

  const int kw0 = kb * kKvBlock + wave * 32;
  const int my_key = kw0 + j;
  const uint16_t* kp = (const uint16_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint16_t* vp = (const uint16_t*)a.v + bi * a.vs.b + g * a.vs.h;

  // K and V rows of this lane's key, as B operands (K^T, V^T) of S and dP.
  V8 kf[NKS], vf[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    if (my_key < a.s_kv) {
      kf[t] = *(const V8*)(kp + (int64_t)my_key * a.ks.s + 16 * t + 8 * h);
      vf[t] = *(const V8*)(vp + (int64_t)my_key * a.vs.s + 16 * t + 8 * h);
    } else {
      kf[t] = V8{};
      vf[t] = V8{};
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const float sl2 = a.scale * kLog2e;
  const int n_qt = (a.s_q + kQTile - 1) / kQTile;
  const int qt0 = CAUSAL ? (kb * kKvBlock) / kQTile : 0;

  for (int hi = 0; hi < Gs; ++hi) {
    const int hq = g * G + sp * Gs + hi;
    const uint16_t* qp = (const uint16_t*)a.q + bi * a.qs.b + hq * a.qs.h;
    const uint16_t* dop = (const uint16_t*)a.dout + bi * a.dos.b + hq * a.dos.h;
    const float* lsep = a.lse + ((int64_t)bi * a.h_q + hq) * a.s_q;
    const float* delp = a.delta + ((int64_t)bi * a.h_q + hq) * a.s_q;
    for (int qt = qt0; qt < n_qt; ++qt) {
      const int q0 = qt * kQTile;
      __syncthreads();
      stage_both<kQTile, D>(qp, a.qs.s, q0, a.s_q, Qs, Qt, tid);
      stage_both<kQTile, D>(dop, a.dos.s, q0, a.s_q, Ds_, Dt, tid);
      if (tid < kQTile) {
        const int qi = q0 + tid;
        lse2s[tid] = qi < a.s_q ? lsep[qi] * kLog2e : 0.f;
        dels[tid] = qi < a.s_q ? delp[qi] : 0.f;
      }
      __syncthreads();
      if (CAUSAL && q0 + kQTile - 1 < kw0) continue;  // every query of the tile precedes this wave's keys

      // S = Q K^T and dP = dO V^T for 32 queries x this lane's key.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const V8 qa = *(const V8*)(&Qs[j * RS + 16 * t + 8 * h]);
        s = T::mfma(qa, kf[t], s);
        const V8 da = *(const V8*)(&Ds_[j * RS + 16 * t + 8 * h]);
        dp = T::mfma(da, vf[t], dp);
      }
      // P and dS; lane owns key my_key, register r owns query q0 + acc_row(r, h).
      uint32_t ppk[8], dspk[8];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int row0 = 8 * r4 + 4 * h;
        const f32x4 l4 = *(const f32x4*)(&lse2s[row0]);
        const f32x4 d4 = *(const f32x4*)(&dels[row0]);
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = q0 + row0 + e;
          const bool ok = qi < a.s_q && my_key < a.s_kv && (!CAUSAL || my_key <= qi);
          const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[4 * r4 + e], sl2, -l4[e])) : 0.f;
          pv[e] = p;
          dsv[e] = p * (dp[4 * r4 + e] - d4[e]);
        }
        ppk[2 * r4] = pack2<T>(pv[0], pv[1]);
        ppk[2 * r4 + 1] = pack2<T>(pv[2], pv[3]);
        dspk[2 * r4] = pack2<T>(dsv[0], dsv[1]);
        dspk[2 * r4 + 1] = pack2<T>(dsv[2], dsv[3]);
      }
      // dV^T += dO^T P ; dK^T += Q^T dS  (16 queries per step)
#pragma unroll
      for (int t2 = 0; t2 < kQTile / 16; ++t2) {
        const V8 pb = __builtin_bit_cast(V8, u32x4{ppk[4 * t2], ppk[4 * t2 + 1], ppk[4 * t2 + 2], ppk[4 * t2 + 3]});
        const V8 sb =
            __builtin_bit_cast(V8, u32x4{dspk[4 * t2], dspk[4 * t2 + 1], dspk[4 * t2 + 2], dspk[4 * t2 + 3]});
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const V8 doa = read_tr_operand<V8>(Dt, TS, db * 32 + j, t2, h);
          dv[db] = T::mfma(doa, pb, dv[db]);
          const V8 qta = read_tr_operand<V8>(Qt, TS, db * 32 + j, t2, h);
          dk[db] = T::mfma(qta, sb, dk[db]);
        }
      }
    }
  }

  if (my_key >= a.s_kv) return;
  if (n_split == 1) {
    uint16_t* dkp = (uint16_t*)a.dk + bi * a.dks.b + g * a.dks.h + (int64_t)my_key * a.dks.s;
    uint16_t* dvp = (uint16_t*)a.dv + bi * a.dvs.b + g * a.dvs.h + (int64_t)my_key * a.dvs.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 wk, wv;
        wk.x = pack2<T>(dk[db][4 * rq] * a.scale, dk[db][4 * rq + 1] * a.scale);
        wk.y = pack2<T>(dk[db][4 * rq + 2] * a.scale, dk[db][4 * rq + 3] * a.scale);
        wv.x = pack2<T>(dv[db][4 * rq], dv[db][4 * rq + 1]);
        wv.y = pack2<T>(dv[db][4 * rq + 2], dv[db][4 * rq + 3]);
        *(u32x2*)(dkp + d0) = wk;
        *(u32x2*)(dvp + d0) = wv;
      }
  } else {
    // fp32 partials: part[2][n_split][b][h_kv][s_kv][D] (dK first, then dV)
    const int64_t plane = (int64_t)a.b * a.h_kv * a.s_kv * D;
    const int64_t off = (int64_t)sp * plane + (((int64_t)bi * a.h_kv + g) * a.s_kv + my_key) * D;
    float* pk = part + off;
    float* pv = part + (int64_t)n_split * plane + off;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        *(f32x4*)(pk + d0) = f32x4{dk[db][4 * rq] * a.scale, dk[db][4 * rq + 1] * a.scale,
                                   dk[db][4 * rq + 2] * a.scale, dk[db][4 * rq + 3] * a.scale};
        *(f32x4*)(pv + d0) = f32x4{dv[db][4 * rq], dv[db][4 * rq + 1], dv[db][4 * rq + 2], dv[db][4 * rq + 3]};
      }
  }
}

// Sums the n_split fp32 partials of dK and dV in split order and rounds them.
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a, int n_split, const float* part) {
  const int64_t plane = (int64_t)a.b * a.h_kv * a.s_kv * a.d;
  const int64_t n4 = plane / 4;
  for (int64_t c = blockIdx.x * 256LL + threadIdx.x; c < 2 * n4; c += (int64_t)gridDim.x * 256) {
    const int which = c >= n4;  // 0: dK, 1: dV
    const int64_t e = (c - which * n4) * 4;
    const float* src = part + (int64_t)which * n_split * plane + e;
    f32x4 acc = *(const f32x4*)src;
    for (int s = 1; s < n_split; ++s) acc += *(const f32x4*)(src + s * plane);
    const int dd = (int)(e % a.d);
    const int64_t row = e / a.d;
    const int key = (int)(row % a.s_kv);
    const int64_t bg = row / a.s_kv;
    const int g = (int)(bg % a.h_kv), bi = (int)(bg / a.h_kv);
    uint16_t* dst = which == 0 ? (uint16_t*)a.dk + bi * a.dks.b + g * a.dks.h + (int64_t)key * a.dks.s
                               : (uint16_t*)a.dv + bi * a.dvs.b + g * a.dvs.h + (int64_t)key * a.dvs.s;
    *(u32x2*)(dst + dd) = u32x2{pack2<T>(acc[0], acc[1]), pack2<T>(acc[2], acc[3])};
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a, int n_qblk) {
  typedef typename T::vec8 V8;
  constexpr int NKS = D / 16, NDB = D / 32, NSB = kKTile / 32;
  constexpr int RS = D + 8, TS = kKTile + 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKTile * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kKTile * RS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int bh_total = a.b * a.h_q;
  const int rank = blockIdx.x / bh_total;
  int slot = blockIdx.x - rank * bh_total;
  if ((bh_total & 7) == 0) {
    const int per = bh_total >> 3;
    slot = (slot & 7) * per + (slot >> 3);
  }
  const int qb = n_qblk - 1 - rank;
  const int bi = slot / a.h_q, hq = slot - (slot / a.h_q) * a.h_q;
  const int g = hq / (a.h_q / a.h_kv);
  const int qblk0 = qb * kQBlock;
  const int q0 = qblk0 + wave * 32;
  const int my_q = q0 + j;

  const uint16_t* qp = (const uint16_t*)a.q + bi * a.qs.b + hq * a.qs.h;
  const uint16_t* dop = (const uint16_t*)a.dout + bi * a.dos.b + hq * a.dos.h;
  const uint16_t* kp = (const uint16_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint16_t* vp = (const uint16_t*)a.v + bi * a.vs.b + g * a.vs.h;

  V8 qf[NKS], df[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    if (my_q < a.s_q) {
      qf[t] = *(const V8*)(qp + (int64_t)my_q * a.qs.s + 16 * t + 8 * h);
      df[t] = *(const V8*)(dop + (int64_t)my_q * a.dos.s + 16 * t + 8 * h);
    } else {
      qf[t] = V8{};
      df[t] = V8{};
    }
  }
  const int64_t row_bh = ((int64_t)bi * a.h_q + hq) * a.s_q;
  const float lse2 = my_q < a.s_q ? a.lse[row_bh + my_q] * kLog2e : 0.f;
  const float dl = my_q < a.s_q ? a.delta[row_bh + my_q] : 0.f;
  const float sl2 = a.scale * kLog2e;

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

  const int kv_end = CAUSAL ? min(a.s_kv, qblk0 + kQBlock) : a.s_kv;
  const int n_tiles = (kv_end + kKTile - 1) / kKTile;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int k0 = tile * kKTile;
    __syncthreads();
    stage_rm<kKTile, D>(kp, a.ks.s, k0, a.s_kv, Ks, tid);
    stage_tr<kKTile, D>(kp, a.ks.s, k0, a.s_kv, Kt, tid);
    stage_rm<kKTile, D>(vp, a.vs.s, k0, a.s_kv, Vs, tid);
    __syncthreads();
    if (CAUSAL && k0 > q0 + 31) continue;

    f32x16 s[NSB], dp[NSB];
#pragma unroll
    for (int nb = 0; nb < NSB; ++nb) {
      s[nb] = f32x16{};
      dp[nb] = f32x16{};
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const V8 ka = *(const V8*)(&Ks[(nb * 32 + j) * RS + 16 * t + 8 * h]);
        s[nb] = T::mfma(ka, qf[t], s[nb]);
        const V8 va = *(const V8*)(&Vs[(nb * 32 + j) * RS + 16 * t + 8 * h]);
        dp[nb] = T::mfma(va, df[t], dp[nb]);
      }
    }
    const bool need_mask = (k0 + kKTile > a.s_kv) || (CAUSAL && k0 + kKTile - 1 > q0);
    uint32_t dspk[NSB][8];
#pragma unroll
    for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float x = s[nb][r + e];
          if (need_mask) {
            const int key = k0 + nb * 32 + acc_row(r + e, h);
            if (key >= a.s_kv || (CAUSAL && key > my_q)) x = -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(fmaf(x, sl2, -lse2));
          ds2[e] = p * (dp[nb][r + e] - dl);
        }
        dspk[nb][r / 2] = pack2<T>(ds2[0], ds2[1]);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t2 = 0; t2 < kKTile / 16; ++t2) {
      const int nb = t2 / 2, base = 4 * (t2 % 2);
      const V8 sb = __builtin_bit_cast(
          V8, u32x4{dspk[nb][base], dspk[nb][base + 1], dspk[nb][base + 2], dspk[nb][base + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const V8 kta = read_tr_operand<V8>(Kt, TS, db * 32 + j, t2, h);
        dq[db] = T::mfma(kta, sb, dq[db]);
      }
    }
  }
  if (my_q < a.s_q) {
    uint16_t* dqp = (uint16_t*)a.dq + bi * a.dqs.b + hq * a.dqs.h + (int64_t)my_q * a.dqs.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 w;
        w.x = pack2<T>(dq[db][4 * rq] * a.scale, dq[db][4 * rq + 1] * a.scale);
        w.y = pack2<T>(dq[db][4 * rq + 2] * a.scale, dq[db][4 * rq + 3] * a.scale);
        *(u32x2*)(dqp + d0) = w;
      }
  }
}

// Number of workgroups a KV head's query-head group is split over: enough
// to put at least 512 dK/dV workgroups in flight when the group allows it.
int choose_split(int b, int h_q, int h_kv, int s_kv) {
  const int G = h_q / h_kv;
  const int64_t base = (int64_t)((s_kv + kKvBlock - 1) / kKvBlock) * b * h_kv;
  int n = 1;
  while (base * n < 512 && 2 * n <= G && G % (2 * n) == 0) n *= 2;
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T, int D>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream, const TimingEvents& te) {
  constexpr int RPB = 256 / (D / 8);
  const bool timed = te.n >= 4;
  const int64_t rows = (int64_t)a.b * a.h_q * a.s_q;
  if (timed) (void)hipEventRecord(te.ev[0], stream);
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, a);
  if (timed) (void)hipEventRecord(te.ev[1], stream);

  const int n_split = choose_split(a.b, a.h_q, a.h_kv, a.s_kv);
  float* part = n_split > 1 ? (float*)((char*)a.delta + align256((size_t)rows * sizeof(float))) : nullptr;
  const int n_kblk = (a.s_kv + kKvBlock - 1) / kKvBlock;
  const dim3 g1(n_kblk * a.b * a.h_kv * n_split);
  if (a.causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), g1, dim3(256), 0, stream, a, n_kblk, n_split, part);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), g1, dim3(256), 0, stream, a, n_kblk, n_split, part);
  if (n_split > 1) {
    const int64_t n4 = (int64_t)a.b * a.h_kv * a.s_kv * D / 4 * 2;
    const int64_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                       stream, a, n_split, (const float*)part);
  }
  if (timed) (void)hipEventRecord(te.ev[2], stream);
  const int n_qblk = (a.s_q + kQBlock - 1) / kQBlock;
  const dim3 g2(n_qblk * a.b * a.h_q);
  if (a.causal)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), g2, dim3(256), 0, stream, a, n_qblk);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), g2, dim3(256), 0, stream, a, n_qblk);
  if (timed) (void)hipEventRecord(te.ev[3], stream);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int b, int h_q, int h_kv, int s_q, int s_kv, int d) {
  size_t bytes = align256((size_t)b * h_q * s_q * sizeof(float));
  const int n_split = choose_split(b, h_q, h_kv, s_kv);
  if (n_split > 1) bytes += 2 * (size_t)n_split * b * h_kv * s_kv * d * sizeof(float);
  return bytes;
}

hipError_t launch_zero_dkdv(const BwdArgs& a, Io io, hipStream_t stream) {
  (void)io;
  const int64_t total = (int64_t)a.b * a.h_kv * a.s_kv * (a.d / 8);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(zero_dkdv_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, Io io, hipStream_t stream, const TimingEvents& te) {
  if (io == Io::BF16)
    return a.d == 64 ? launch_all<Bf16T, 64>(a, stream, te) : launch_all<Bf16T, 128>(a, stream, te);
  return a.d == 64 ? launch_all<F16T, 64>(a, stream, te) : launch_all<F16T, 128>(a, stream, te);
}

}  // namespace sdpa
