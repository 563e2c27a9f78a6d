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
// Kernels (all atomic-free and deterministic), in launch order:
//  1. dQ:     Q-stationary, laid out like the forward: each lane owns one
//     query column of S^T = K Q^T; dQ^T += K^T dS^T with K^T read from the
//     row-major K tile through ds_read_b64_tr_b16. It also forms
//     D = rowsum(dO * O) of its rows (fp32) and leaves it in the workspace.
//  2. dK/dV:  KV-stationary. A workgroup owns 256 keys (32 per wave) whose K
//     and V rows stay in LDS; it loops over the query heads of its group and
//     over 32-row query tiles staged row-major in LDS, read both as row
//     operands and, through ds_read_b64_tr_b16, as transposed ones.
//     Each lane owns one key column of S = Q K^T, so P and dS are directly the
//     B operands of dV^T += dO^T P and dK^T += Q^T dS.
//     When a GQA/MQA group would leave the GPU underfilled, the group's query
//     heads are split over several workgroups that write fp32 partials.
//     At d = 128 without score modifiers the same block runs as 4 waves of
//     64 keys (bwd_dkdv64_kernel): one wave per SIMD, AGPR accumulators,
//     each LDS operand read feeding two MFMAs, the wave's K rows in
//     registers and two query-tile buffers (one barrier per tile).
//  3. reduce: sums the partials of the splits in a fixed order.
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

constexpr int kKvBlock = 256;  // keys per dK/dV workgroup (8 waves x 32)
constexpr int kQTile = 32;     // query rows per dK/dV inner step
// Waves (of 32 query rows) per dQ workgroup: at d = 128, 8 waves (one
// workgroup per CU) share each K/V tile staging; at d = 64 a 32-key tile is
// only 256 16-byte chunks, one per thread of 4 waves.
constexpr int dq_waves(int d) { return d == 128 ? 8 : 4; }
constexpr int kKTile = 32;     // keys per dQ inner step

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

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// Chunk swizzle of the row-major LDS tiles read both as rows and through
// transposed reads (the Q and dO tiles of the dK/dV kernel, the K and V tiles
// of the dQ kernel; no row padding): 16-byte chunk c of row r sits at
// position c ^ bswz<D>(r). Two access patterns meet it. A 16-byte row read
// (MFMA row operand) by 16 consecutive lanes touches chunk c of 16
// consecutive rows; a transposed read (ds_read_b64_tr_b16) by 32 lanes
// touches 4 consecutive rows x 4 consecutive chunks. With 64 banks of 4 bytes,
// D = 128 (one row per 256 bytes) needs bswz to take 16 distinct values over
// 16 rows and to give rows 4k..4k+3 distinct values in bits 2-3; D = 64 (two
// rows per 256 bytes) needs 8 distinct values over the even (and the odd)
// rows and distinct bit 2 for rows 4k and 4k+2. Both choices below do that.
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 128 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Lane offsets of the transposed operand reads from a bswz tile of D columns:
// lane (column 32 db + l % 32, half h) receives rows 16 t + 4 h + 0..3 (lo) and
// 16 t + 8 + 4 h + 0..3 (hi), the rows key_of() assigns to the accumulator
// registers of S. bswz is invariant under +16 rows but not under +8, so the
// lo and hi reads carry their own offsets.
template <int D>
struct TrLaneB {
  int lo[D / 32], hi[D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int i = lane & 15, grp = lane >> 4, h = lane >> 5;
    const int row = 4 * h + (i >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * (grp & 1) + 4 * (i & 3);
      lo[db] = row * D + (((col >> 3) ^ bswz<D>(row)) * 8) + 4 * ((col >> 2) & 1);
      hi[db] = (row + 8) * D + (((col >> 3) ^ bswz<D>(row + 8)) * 8) + 4 * ((col >> 2) & 1);
    }
  }
  template <typename V8>
  __device__ __forceinline__ V8 tr(const uint16_t* tile, int db, int t) const {
    const u32x2 l = ds_read_tr16(&tile[lo[db] + 16 * t * D]);
    const u32x2 u = ds_read_tr16(&tile[hi[db] + 16 * t * D]);
    return __builtin_bit_cast(V8, u32x4{l.x, l.y, u.x, u.y});
  }
};

// A tile of R rows x D 16-bit elements in flight as 16-byte row chunks
// (NT threads), written to LDS row-major in the bswz layout. Buffer loads;
// rows past the descriptor's bytes read as zero.
template <int R, int D, int NT>
struct BswzTile {
  static constexpr int CH = D / 8;
  static constexpr int NC = R * CH / NT;
  static_assert(NC * NT == R * CH, "tile / thread mismatch");
  u32x4 v[NC];
  uint32_t off[NC];
  int dst[NC];
  int64_t stride;

  __device__ __forceinline__ void init(int64_t row_stride, int tid) {
    stride = row_stride;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = tid + NT * i;
      const int r = c / CH, cc = c % CH;
      off[i] = (uint32_t)(r * row_stride * 2 + cc * 16);
      dst[i] = r * D + ((cc ^ bswz<D>(r)) * 8);
    }
  }
  // Loads rows row0.. with a descriptor that allows `bytes` bytes from row0
  // (tile_bytes; 0: every load returns zeros and reads no memory).
  __device__ __forceinline__ void load(const uint16_t* base, int row0, uint32_t bytes) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + row0 * stride, bytes);
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = buf_load16(rs, off[i]);
  }
  __device__ __forceinline__ void store(uint16_t* tile) const {
#pragma unroll
    for (int i = 0; i < NC; ++i) *(u32x4*)(&tile[dst[i]]) = v[i];
  }
};

// KV-stationary dK/dV. A workgroup has 8 waves (two per SIMD) and 256 keys;
// wave w owns keys 32 w .. 32 w + 31 of the block and accumulates their dK^T,
// dV^T in VGPRs. The block's K and V rows sit in LDS for the whole kernel
// (132 KB at d = 128); the workgroup walks (query head of its group slice,
// 32-row query tile) pairs in order, staging each Q / dO tile (and its LSE
// and D values) in one LDS buffer; the next pair's tile is loaded into
// registers while the current one is computed. The transposed Q^T / dO^T
// operands of dK and dV are read from the same row-major tiles with
// ds_read_b64_tr_b16.
template <typename T, int D, bool CAUSAL, int MOD>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a, int n_kblk, int n_split, float* part) {
  typedef typename T::vec8 V8;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int NT = 512;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int KVC = kKvBlock * CH / NT;     // K (and V) block chunks per thread
  constexpr int QCH = kQTile * CH;            // chunks of one Q (or dO) tile
  constexpr int QPT = (QCH + NT - 1) / NT;    // of which each thread stages up to QPT
  static_assert(KVC * NT == kKvBlock * CH, "tile / thread mismatch");
  // K/V block: row r holds K row r, then V row r, then 16 bytes of padding.
  // The pitch is 16 bytes past a multiple of 256, so 16 lanes reading one
  // 16-byte column chunk of 16 consecutive rows hit 16 distinct bank groups,
  // and every K and V operand read of a lane is one base plus an immediate.
  constexpr int KVP = 2 * D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t KV[kKvBlock * KVP];
  // Q tile, then the dO tile, both in the bswz layout: the dO operands sit at
  // an immediate offset from the Q operands.
  __shared__ __attribute__((aligned(16))) uint16_t QD[2 * kQTile * D];
  uint16_t* const Qs = QD;
  uint16_t* const Ds_ = QD + kQTile * D;
  __shared__ __attribute__((aligned(16))) float lse2s[kQTile];
  __shared__ __attribute__((aligned(16))) float dels[kQTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int n_slots = a.b * a.h_kv * n_split;
  // Linear id -> (key block, slot); causal: key block 0 (the most query tiles) first.
  // The n_split workgroups of one KV group load the same K/V block: one XCD.
  const int kb = blockIdx.x / n_slots;
  const int slot = xcd_slot(blockIdx.x - kb * n_slots, n_slots, n_split);
  const int sp = slot % n_split;
  const int bg = slot / n_split;
  const int g = bg % a.h_kv, bi = bg / a.h_kv;
  const int G = a.h_q / a.h_kv, Gs = G / n_split;
  (void)n_kblk;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const int kw0 = kb * kKvBlock + wave * 32;
  const int my_key = kw0 + j;
  const uint16_t* kp = (const uint16_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint16_t* vp = (const uint16_t*)a.v + bi * a.vs.b + g * a.vs.h;

  // Stage the block's K and V rows once (keys at or past lk read as zero).
  {
    const int k0 = kb * kKvBlock;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + (int64_t)k0 * a.ks.s, tile_bytes(k0, L.lk, a.ks.s, D, 2));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + (int64_t)k0 * a.vs.s, tile_bytes(k0, L.lk, a.vs.s, D, 2));
#pragma unroll
    for (int i = 0; i < KVC; ++i) {
      const int c = tid + NT * i;
      const int r = c / CH, cc = c % CH;
      const int dst = r * KVP + cc * 8;
      *(u32x4*)(&KV[dst]) = buf_load16(kr, (uint32_t)(r * a.ks.s * 2 + cc * 16));
      *(u32x4*)(&KV[dst + D]) = buf_load16(vr, (uint32_t)(r * a.vs.s * 2 + cc * 16));
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const float sl2 = a.scale * kLog2e;
  // Query tiles of valid rows that can see a key of this block: row i sees
  // key j iff j <= i + off, so causal rows start at (block start) - off. A
  // block made only of keys past lk has no work (its dK, dV are zero).
  const int n_qt = (L.lq + kQTile - 1) / kQTile;
  const int qt0 = CAUSAL ? min(n_qt, max(0, kb * kKvBlock - L.off) / kQTile) : 0;
  const int nq = kb * kKvBlock >= L.lk ? 0 : n_qt - qt0;
  const int n_it = Gs * nq;
  const int hq_base = g * G + sp * Gs;

  // Per-lane LDS offsets, loop-invariant: this lane's row of the Q / dO tile
  // (row j), chunk 2 t + h, and of the K / V block (row 32 wave + j).
  int rowoff_q[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) rowoff_q[t] = j * D + (((2 * t + h) ^ bswz<D>(j)) * 8);
  const int kvoff = (wave * 32 + j) * KVP + 8 * h;
  TrLaneB<D> trl;
  trl.init(lane);

  // Q / dO tile staging: chunk c = tid + NT i (c < QCH) is row c / CH, column
  // chunk c % CH. (When every thread stages, no branch guards the loads: the
  // unconditional form schedules measurably better.)
  uint32_t qoff[QPT], doff[QPT];
  int sdst[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = tid + NT * i, sr = c / CH, scc = c % CH;
    qoff[i] = (uint32_t)(sr * a.qs.s * 2 + scc * 16);
    doff[i] = (uint32_t)(sr * a.dos.s * 2 + scc * 16);
    sdst[i] = sr * D + ((scc ^ bswz<D>(sr)) * 8);
  }
  u32x4 qreg[QPT], dreg[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) qreg[i] = dreg[i] = u32x4{0, 0, 0, 0};
  // LSE and D of the next tile's rows, raw as loaded: nothing uses them before
  // they are staged at the next iteration, so the loads stay in flight through
  // this tile's compute (a use here would make the wave wait for every load
  // of the prefetch, and the whole workgroup for that wave at the barrier).
  float lreg = 0.f, creg = 0.f;
  bool lvalid = false;
  auto load_tile = [&](int it) {
    const int hq = hq_base + it / nq;
    const int q0 = (qt0 + it % nq) * kQTile;
    const uint16_t* qp = (const uint16_t*)a.q + bi * a.qs.b + hq * a.qs.h + (int64_t)q0 * a.qs.s;
    const uint16_t* dop = (const uint16_t*)a.dout + bi * a.dos.b + hq * a.dos.h + (int64_t)q0 * a.dos.s;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp, tile_bytes(q0, L.lq, a.qs.s, D, 2));
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dop, tile_bytes(q0, L.lq, a.dos.s, D, 2));
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (QCH % NT == 0 || tid + NT * i < QCH) {  // rows at or past lq read as zero
        qreg[i] = buf_load16(qr, qoff[i]);
        dreg[i] = buf_load16(dr, doff[i]);
      }
    if (tid < kQTile) {  // rows past lq read row lq - 1 (any valid row) and are zeroed when staged
      const int qi = q0 + tid;
      lvalid = qi < L.lq;
      const int64_t row = ((int64_t)bi * a.h_q + hq) * a.s_q + min(qi, L.lq - 1);
      lreg = a.lse[row];
      creg = a.delta[row];
    }
  };

  if (n_it > 0) load_tile(0);
  for (int it = 0; it < n_it; ++it) {
    const int q0 = (qt0 + it % nq) * kQTile;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (QCH % NT == 0 || tid + NT * i < QCH) {
        *(u32x4*)(&Qs[sdst[i]]) = qreg[i];
        *(u32x4*)(&Ds_[sdst[i]]) = dreg[i];
      }
    if (tid < kQTile) {
      // A row that sees no key has LSE = -inf; all its scores are masked, and
      // 0 here keeps exp2(-inf - lse) at 0 instead of NaN.
      lse2s[tid] = (lvalid && lreg != -INFINITY) ? lreg * kLog2e : 0.f;
      dels[tid] = lvalid ? creg : 0.f;
    }
    if (it + 1 < n_it) load_tile(it + 1);
    __syncthreads();  // this tile is in LDS
    // Tiles whose queries all precede this wave's keys add nothing.
    if (CAUSAL && q0 + kQTile - 1 + L.off < kw0) continue;

    // S = Q K^T and dP = dO V^T for 32 queries x this lane's key.
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < NKS; ++t) {
      s = T::mfma(*(const V8*)(&Qs[rowoff_q[t]]), *(const V8*)(&KV[kvoff + 16 * t]), s);
      dp = T::mfma(*(const V8*)(&Ds_[rowoff_q[t]]), *(const V8*)(&KV[kvoff + D + 16 * t]), dp);
    }
    if constexpr (MOD == kModNone) {
      // Operand reads (two per MFMA) issued kLookK MFMAs ahead. Same-box
      // sweep of the backward: none 1.906 ms, 2: 1.883, 3: 1.891, 4: 1.892,
      // 5: 1.874; scheduling the dV/dK transposed reads as well: no gain.
      constexpr int kLookK = 5;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLookK, 0);
#pragma unroll
      for (int i = 0; i < 2 * NKS - kLookK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kLookK, 0);
    }
    // P and dS; lane owns key my_key, register r owns query q0 + acc_row(r, h).
    const bool need_mask = (q0 + kQTile > L.lq) || (kw0 + 32 > L.lk) || (CAUSAL && q0 + L.off < kw0 + 31);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + acc_row(r, h);
        if (qi >= L.lq || my_key >= L.lk || (CAUSAL && my_key > qi + L.off)) s[r] = -INFINITY;
      }
    }
    // Score modifiers of this query head (log2 units), applied per row group below.
    const int hq_it = hq_base + it / nq;
    const float slope2 = (MOD && a.mod.slopes != nullptr) ? a.mod.slopes[hq_it] * kLog2e : 0.f;
    const char* bias_bh = (MOD == kModAll && a.mod.bias != nullptr)
                              ? (const char*)a.mod.bias + (bi * a.mod.bb + hq_it * a.mod.bh) * (a.mod.bias_f32 ? 4 : 2)
                              : nullptr;
    // Dropout keep bytes of this lane's key: byte e of kb[r4] is query q0 + 8 r4 + 4 h + e.
    // The four lanes of a key quad share the tile's four blocks (one per r4):
    // lane t draws block r4 = t, regroups its bytes per key and the quad
    // trades them.
    u32x4 kb = u32x4{0u, 0u, 0u, 0u};
    if (MOD >= kModDrop && a.mod.drop_k8 < 256) {
      const uint32_t t = (uint32_t)(lane & 3);
      const u32x4 w = drop_words((uint32_t)my_key >> 2, (uint32_t)(q0 + 8 * t + 4 * h) >> 2,
                                 (uint32_t)(bi * a.h_q + hq_it), a.mod.offset, a.mod.seed_lo, a.mod.seed_hi);
      kb = quad_transpose(bytes_transpose4(w), lane);
    }
    uint32_t ppk[8], dspk[8];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int row0 = 8 * r4 + 4 * h;
      const f32x4 l4 = *(const f32x4*)(&lse2s[row0]);
      const f32x4 d4 = *(const f32x4*)(&dels[row0]);
      float pv[4], dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float madd = 0.f;
        if (MOD) {
          const int qi = q0 + row0 + e;
          const void* brow = (bias_bh != nullptr && qi < a.s_q)
                                 ? (const void*)(bias_bh + (int64_t)qi * a.mod.bs * (a.mod.bias_f32 ? 4 : 2))
                                 : nullptr;
          const float bv = MOD == kModAll ? bias1<T>(brow, a.mod.bias_f32, my_key, a.s_kv) : 0.f;
          madd = fmaf(bv, kLog2e, -slope2 * fabsf((float)(qi + L.off - my_key)));
        }
        const float p = __builtin_amdgcn_exp2f(fmaf(s[4 * r4 + e], sl2, madd - l4[e]));
        if (MOD >= kModDrop) {  // dV takes P Z (Z's scale applied at the end); dS = P (Z dP - D)
          const bool keep = drop_keep(kb[r4], e, a.mod.drop_k8);
          pv[e] = keep ? p : 0.f;
          dsv[e] = p * ((keep ? a.mod.drop_scale * dp[4 * r4 + e] : 0.f) - d4[e]);
        } else {
          pv[e] = p;
          dsv[e] = p * (dp[4 * r4 + e] - d4[e]);
        }
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
        dv[db] = T::mfma(trl.template tr<V8>(Ds_, db, t2), pb, dv[db]);
        dk[db] = T::mfma(trl.template tr<V8>(Qs, db, t2), sb, dk[db]);
      }
    }
  }

  if (my_key >= a.s_kv) return;
  const float vsc = MOD >= kModDrop ? a.dv_scale * a.mod.drop_scale : a.dv_scale;  // dV = (P Z)^T dO, Z = keep * drop_scale
  if (n_split == 1) {
    uint16_t* dkp = (uint16_t*)a.dk + bi * a.dks.b + g * a.dks.h + (int64_t)my_key * a.dks.s;
    uint16_t* dvp = (uint16_t*)a.dv + bi * a.dvs.b + g * a.dvs.h + (int64_t)my_key * a.dvs.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 wk, wv;
        wk.x = pack2<T>(dk[db][4 * rq] * a.dk_scale, dk[db][4 * rq + 1] * a.dk_scale);
        wk.y = pack2<T>(dk[db][4 * rq + 2] * a.dk_scale, dk[db][4 * rq + 3] * a.dk_scale);
        wv.x = pack2<T>(dv[db][4 * rq] * vsc, dv[db][4 * rq + 1] * vsc);
        wv.y = pack2<T>(dv[db][4 * rq + 2] * vsc, dv[db][4 * rq + 3] * vsc);
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
        *(f32x4*)(pk + d0) = f32x4{dk[db][4 * rq] * a.dk_scale, dk[db][4 * rq + 1] * a.dk_scale,
                                   dk[db][4 * rq + 2] * a.dk_scale, dk[db][4 * rq + 3] * a.dk_scale};
        *(f32x4*)(pv + d0) =
            f32x4{dv[db][4 * rq] * vsc, dv[db][4 * rq + 1] * vsc, dv[db][4 * rq + 2] * vsc, dv[db][4 * rq + 3] * vsc};
      }
  }
}

// KV-stationary dK/dV at d = 128 without score modifiers, one wave per SIMD.
// A workgroup has 4 waves and the same 256-key block as bwd_dkdv_kernel, but
// wave w owns 64 keys (two 32-key halves): every Q, dO row operand and every
// Q^T, dO^T transposed operand read from LDS feeds two MFMAs, one per half,
// and the dK^T / dV^T accumulators (256 registers) live in AGPRs, where the
// vector work of the same wave can issue beside the MFMAs that update them.
// The wave's K rows stay in registers for the whole kernel (64 VGPRs, the B
// operands of S = Q K^T); only the V rows sit in LDS, which leaves room for
// two Q/dO tile buffers: the next tile is staged into the other buffer while
// the current one is computed, one barrier per tile. With one wave per SIMD
// nothing hides a pause, so the tile body is a fixed slot schedule (four
// phases of 16 MFMAs, operands read four slots ahead).
template <typename T, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv64_kernel(BwdArgs a, int n_split, float* part) {
  typedef typename T::vec8 V8;
  constexpr int D = 128, NKS = D / 16, NDB = D / 32;
  constexpr int NT = 256;
  constexpr int CH = D / 8;
  constexpr int KVC = kKvBlock * CH / NT;
  constexpr int QCH = kQTile * CH;
  constexpr int QPT = QCH / NT;
  constexpr int TB = 2 * kQTile * D;  // one tile buffer: Q rows, then dO rows
  static_assert(KVC * NT == kKvBlock * CH && QPT * NT == QCH, "tile / thread mismatch");
  // V rows padded by 16 bytes: the 16 rows a lane group reads start 4 banks apart.
  constexpr int VP = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kKvBlock * VP];
  __shared__ __attribute__((aligned(16))) uint16_t QD[2 * TB];
  // -LSE log2 e and D of a tile's rows, per buffer and per wave (lane l holds
  // row l % 32): each wave writes and reads its own copy.
  __shared__ __attribute__((aligned(16))) float nls[2][4][64];
  __shared__ __attribute__((aligned(16))) float dls[2][4][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int n_slots = a.b * a.h_kv * n_split;
  const int kb = blockIdx.x / n_slots;
  const int slot = xcd_slot(blockIdx.x - kb * n_slots, n_slots, n_split);
  const int sp = slot % n_split;
  const int bg = slot / n_split;
  const int g = bg % a.h_kv, bi = bg / a.h_kv;
  const int G = a.h_q / a.h_kv, Gs = G / n_split;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const int kw0 = kb * kKvBlock + wave * 64;  // this wave's keys: kw0 .. kw0 + 63
  const int key0 = kw0 + j, key1 = key0 + 32;
  const uint16_t* kp = (const uint16_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint16_t* vp = (const uint16_t*)a.v + bi * a.vs.b + g * a.vs.h;
  // The wave's K rows (key kw0 + 32 hf + j, elements 16 t + 8 h .. + 7 in
  // lane (j, h)) straight into registers; the block's V rows into LDS. Keys
  // at or past lk read as zero.
  V8 kf[2][NKS];
  {
    const int k0 = kb * kKvBlock;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + (int64_t)k0 * a.ks.s, tile_bytes(k0, L.lk, a.ks.s, D, 2));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + (int64_t)k0 * a.vs.s, tile_bytes(k0, L.lk, a.vs.s, D, 2));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int t = 0; t < NKS; ++t)
        kf[hf][t] = __builtin_bit_cast(
            V8, buf_load16(kr, (uint32_t)((wave * 64 + 32 * hf + j) * a.ks.s * 2 + (16 * t + 8 * h) * 2)));
#pragma unroll
    for (int i = 0; i < KVC; ++i) {
      const int c = tid + NT * i;
      const int r = c / CH, cc = c % CH;
      *(u32x4*)(&Vs[r * VP + cc * 8]) = buf_load16(vr, (uint32_t)(r * a.vs.s * 2 + cc * 16));
    }
  }
  f32x16 dk0[NDB], dk1[NDB], dv0[NDB], dv1[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dk0[i] = dk1[i] = dv0[i] = dv1[i] = f32x16{};
  const float sl2 = a.scale * kLog2e;
  const int n_qt = (L.lq + kQTile - 1) / kQTile;
  const int qt0 = CAUSAL ? min(n_qt, max(0, kb * kKvBlock - L.off) / kQTile) : 0;
  const int nq = kb * kKvBlock >= L.lk ? 0 : n_qt - qt0;
  const int n_it = Gs * nq;
  const int hq_base = g * G + sp * Gs;

  int rowoff_q[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) rowoff_q[t] = j * D + (((2 * t + h) ^ bswz<D>(j)) * 8);
  const int voff = (wave * 64 + j) * VP + 8 * h;  // half 1: + 32 rows, an immediate
  TrLaneB<D> trl;
  trl.init(lane);

  uint32_t qoff[QPT], doff[QPT];
  int sdst[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = tid + NT * i, sr = c / CH, scc = c % CH;
    qoff[i] = (uint32_t)(sr * a.qs.s * 2 + scc * 16);
    doff[i] = (uint32_t)(sr * a.dos.s * 2 + scc * 16);
    sdst[i] = sr * D + ((scc ^ bswz<D>(sr)) * 8);
  }
  // The tile walk: (query head, query tile) pairs, tiles qt0 .. n_qt - 1 of
  // each head of the slice. The next tile to load is tracked by running
  // addresses (Q and dO tile bytes, LSE / D row of its first query) that move
  // one tile down the head, or from a head's last tile to the next head's
  // tile qt0: no index arithmetic per tile.
  const int64_t tq = (int64_t)kQTile * a.qs.s * 2, td = (int64_t)kQTile * a.dos.s * 2;
  const int64_t wq = (int64_t)a.qs.h * 2 - (int64_t)(nq - 1) * tq;
  const int64_t wd = (int64_t)a.dos.h * 2 - (int64_t)(nq - 1) * td;
  const int64_t wr = (int64_t)a.s_q - (int64_t)(nq - 1) * kQTile;
  const char* qn = (const char*)a.q + (bi * a.qs.b + hq_base * a.qs.h + (int64_t)qt0 * kQTile * a.qs.s) * 2;
  const char* dn = (const char*)a.dout + (bi * a.dos.b + hq_base * a.dos.h + (int64_t)qt0 * kQTile * a.dos.s) * 2;
  int64_t rn = ((int64_t)bi * a.h_q + hq_base) * a.s_q + qt0 * kQTile;
  // Bytes a tile may read: all its rows, or up to row lq - 1 in a head's
  // last tile (rows past it read as zero).
  const uint32_t qfull = tile_bytes(0, kQTile, a.qs.s, D, 2), dfull = tile_bytes(0, kQTile, a.dos.s, D, 2);
  const uint32_t qlast = tile_bytes((n_qt - 1) * kQTile, L.lq, a.qs.s, D, 2);
  const uint32_t dlast = tile_bytes((n_qt - 1) * kQTile, L.lq, a.dos.s, D, 2);
  u32x4 qreg[QPT], dreg[QPT];
  float lreg = 0.f, creg = 0.f;
  bool lvalid = false;
  int l_qt = qt0, c_qt = qt0;  // query tile of the next load, of the next computed tile
  // Loading a tile takes four steps, issued in separate MFMA slots: buffer
  // descriptors (zero bytes past the last tile, so those loads return zeros
  // and touch no memory), the Q / dO loads, the LSE / D loads of row
  // min(lane % 32, last valid row), the cursor step.
  __amdgpu_buffer_rsrc_t rq, rd, rl, rc;
  int lq0 = 0;
  auto tile_rsrc = [&](bool more) {
    const bool last = l_qt == n_qt - 1;
    lq0 = l_qt * kQTile;
    rq = make_rsrc(qn, more ? (last ? qlast : qfull) : 0u);
    rd = make_rsrc(dn, more ? (last ? dlast : dfull) : 0u);
    rl = make_rsrc(a.lse + rn, more ? 4u * kQTile : 0u);
    rc = make_rsrc(a.delta + rn, more ? 4u * kQTile : 0u);
  };
  auto tile_loads = [&]() {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      qreg[i] = buf_load16(rq, qoff[i]);
      dreg[i] = buf_load16(rd, doff[i]);
    }
  };
  auto tile_stats = [&](bool more) {
    const int l = lane & 31;
    lvalid = more && lq0 + l < L.lq;
    const uint32_t o = (uint32_t)min(l, max(L.lq - 1 - lq0, 0)) * 4u;
    lreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, o, 0, 0));
    creg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, o, 0, 0));
  };
  auto tile_next = [&]() {
    const bool last = l_qt == n_qt - 1;
    l_qt = last ? qt0 : l_qt + 1;
    qn += last ? wq : tq;
    dn += last ? wd : td;
    rn += last ? wr : (int64_t)kQTile;
  };

  // Registers (the next tile) -> tile buffer b. A row past lq, or one that
  // sees no key, gets -LSE = -inf: its weights are exp2(-inf) = 0 whatever its
  // (zero or masked) scores.
  auto stage_regs = [&](int b) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      *(u32x4*)(&QD[b * TB + sdst[i]]) = qreg[i];
      *(u32x4*)(&QD[b * TB + kQTile * D + sdst[i]]) = dreg[i];
    }
    // (Selects, not && : a short-circuit becomes a branch that would split
    // the slot schedule this runs in.)
    const bool ok = lvalid & (lreg != -INFINITY);
    nls[b][wave][lane] = ok ? -lreg * kLog2e : -INFINITY;
    dls[b][wave][lane] = lvalid ? creg : 0.f;
  };
  // The loop is unrolled by the two buffers (their LDS addresses become
  // immediates) and runs an even number of tiles: a last padding tile has
  // zero-byte loads, so it adds nothing (Q = dO = 0, -LSE = -inf).
  const int n_it2 = (n_it + 1) & ~1;
  if (n_it2 > 0) {
    tile_rsrc(true);
    tile_loads();
    tile_stats(true);
    tile_next();
    stage_regs(0);
    tile_rsrc(n_it > 1);
    tile_loads();
    tile_stats(n_it > 1);
    tile_next();
  }
  auto step = [&](const int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* const Qs = QD + buf * TB;
    const uint16_t* const Ds_ = Qs + kQTile * D;
    const int q0 = c_qt * kQTile;
    c_qt = c_qt == n_qt - 1 ? qt0 : c_qt + 1;
    // Buffer `buf` holds tile it; every wave is done with tile it - 1, whose
    // buffer takes tile it + 1 in phase D.
    __syncthreads();
    const bool more = it + 2 < n_it;
    // A tile whose queries all precede this wave's keys is computed anyway,
    // fully masked (it adds zeros): the SIMD has no other wave to give the
    // time to, and a branch around the accumulation makes the register
    // allocator move the AGPR accumulators through VGPRs.

    // Four phases of 16 MFMA slots each; a scheduling fence closes every
    // slot, so the vector work placed in a slot issues beside that slot's
    // MFMA, and every LDS operand is read kLA slots before its MFMA:
    //   A: S = Q K^T (K from registers; both key halves share each Q read)
    //   B: dP = dO V^T, beside it P = exp2(S scale log2 e - LSE log2 e)
    //   C: dV^T += dO^T P (AGPR accumulators), beside it dS = P (dP - D)
    //   D: dK^T += Q^T dS, beside it the staging of tile it + 1 (loaded a
    //      step earlier) and the loads of tile it + 2
    constexpr int kLA = 4;
    const bool need_mask = (kw0 + 64 > L.lk) || (CAUSAL && q0 + L.off < kw0 + 63);
    f32x16 sc[2] = {f32x16{}, f32x16{}}, dpc[2] = {f32x16{}, f32x16{}};
    V8 ra[8], rb[2][8];   // phase A / B row operands: Q or dO (shared), V per half
    f32x4 nl4[4], d4[4];  // -LSE log2 e and D of the lane's 16 query rows
    float pf[2][16];
    uint32_t pk[2][8], sk[2][8];
    // Row-operand reads of slot m of phases A (m < 16) and B (m >= 16).
    auto read_ab = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 32) {
        constexpr int t = (m & 15) >> 1, hf = m & 1;
        const uint16_t* tile = m < 16 ? Qs : Ds_;
        if constexpr (hf == 0) ra[t] = *(const V8*)(&tile[rowoff_q[t]]);
        if constexpr (m >= 16) rb[hf][t] = *(const V8*)(&Vs[voff + (hf ? 32 * VP : 0) + 16 * t]);
      }
    };
    static_for<kLA>([&](auto mc) { read_ab(mc); });
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) nl4[r4] = *(const f32x4*)(&nls[buf][wave][8 * r4 + 4 * h]);
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value, t = m >> 1, hf = m & 1;
      sc[hf] = T::mfma(ra[t], kf[hf][t], sc[hf]);
      read_ab(std::integral_constant<int, m + kLA>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if (need_mask) {
      // Key k is hidden from row qi iff k > qi + off (causal) or k >= lk; with
      // qi = q0 + 4 h + c, c = acc_row(r, 0), that is e > c for a per-half e.
      const int qb = q0 + L.off + 4 * h;
      const int e0 = key0 >= L.lk ? 0x7fffffff : CAUSAL ? key0 - qb : -0x7fffffff;
      const int e1 = key1 >= L.lk ? 0x7fffffff : CAUSAL ? key1 - qb : -0x7fffffff;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (e0 > acc_row(r, 0)) sc[0][r] = -INFINITY;
        if (e1 > acc_row(r, 0)) sc[1][r] = -INFINITY;
      }
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) d4[r4] = *(const f32x4*)(&dls[buf][wave][8 * r4 + 4 * h]);
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value, t = m >> 1, hf = m & 1;
      dpc[hf] = T::mfma(ra[t], rb[hf][t], dpc[hf]);
      read_ab(std::integral_constant<int, m + 16 + kLA>{});
      // P: two weights per slot, half ph, elements 2 w and 2 w + 1.
      constexpr int ph = m >> 3, w = m & 7, r = 2 * w;
      pf[ph][r] = __builtin_amdgcn_exp2f(fmaf(sc[ph][r], sl2, nl4[r >> 2][r & 3]));
      pf[ph][r + 1] = __builtin_amdgcn_exp2f(fmaf(sc[ph][r + 1], sl2, nl4[(r + 1) >> 2][(r + 1) & 3]));
      pk[ph][w] = pack2<T>(pf[ph][r], pf[ph][r + 1]);
      __builtin_amdgcn_sched_barrier(0);
    });
    // Transposed operands of phases C (dO^T) and D (Q^T), slot m: (t2, db) =
    // (m / 8, (m / 2) % 4) of each phase, shared by the two key halves.
    V8 ta[2][2][NDB];
    auto read_cd = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 32 && (m & 1) == 0) {
        constexpr int ph = m >> 4, t2 = (m & 15) >> 3, db = (m >> 1) & 3;
        ta[ph][t2][db] = trl.template tr<V8>(ph ? Qs : Ds_, db, t2);
      }
    };
    static_for<kLA>([&](auto mc) { read_cd(mc); });
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value, t2 = m >> 3, db = (m >> 1) & 3, hf = m & 1;
      const V8 pb = __builtin_bit_cast(V8, u32x4{pk[hf][4 * t2], pk[hf][4 * t2 + 1], pk[hf][4 * t2 + 2], pk[hf][4 * t2 + 3]});
      if (hf) mfma_acc<T>(dv1[db], ta[0][t2][db], pb);
      else mfma_acc<T>(dv0[db], ta[0][t2][db], pb);
      read_cd(std::integral_constant<int, m + kLA>{});
      // dS: two per slot.
      constexpr int ph = m >> 3, w = m & 7, r = 2 * w;
      const float g0 = pf[ph][r] * (dpc[ph][r] - d4[r >> 2][r & 3]);
      const float g1 = pf[ph][r + 1] * (dpc[ph][r + 1] - d4[(r + 1) >> 2][(r + 1) & 3]);
      sk[ph][w] = pack2<T>(g0, g1);
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value, t2 = m >> 3, db = (m >> 1) & 3, hf = m & 1;
      const V8 sb = __builtin_bit_cast(V8, u32x4{sk[hf][4 * t2], sk[hf][4 * t2 + 1], sk[hf][4 * t2 + 2], sk[hf][4 * t2 + 3]});
      if (hf) mfma_acc<T>(dk1[db], ta[1][t2][db], sb);
      else mfma_acc<T>(dk0[db], ta[1][t2][db], sb);
      read_cd(std::integral_constant<int, m + 16 + kLA>{});
      if constexpr (m == 8) stage_regs(buf ^ 1);
      if constexpr (m == 9) tile_rsrc(more);
      if constexpr (m == 10) tile_loads();
      if constexpr (m == 11) tile_stats(more);
      if constexpr (m == 12) tile_next();
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int it = 0; it < n_it2; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    step(it + 1, std::integral_constant<int, 1>{});
  }
  mfma_acc_drain(dk0, dk1, dv0, dv1);

  const float vsc = a.dv_scale;
  auto store_keys = [&](const f32x16 (&dk)[NDB], const f32x16 (&dv)[NDB], int my_key) {
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
          wk.x = pack2<T>(dk[db][4 * rq] * a.dk_scale, dk[db][4 * rq + 1] * a.dk_scale);
          wk.y = pack2<T>(dk[db][4 * rq + 2] * a.dk_scale, dk[db][4 * rq + 3] * a.dk_scale);
          wv.x = pack2<T>(dv[db][4 * rq] * vsc, dv[db][4 * rq + 1] * vsc);
          wv.y = pack2<T>(dv[db][4 * rq + 2] * vsc, dv[db][4 * rq + 3] * vsc);
          *(u32x2*)(dkp + d0) = wk;
          *(u32x2*)(dvp + d0) = wv;
        }
    } else {
      const int64_t plane = (int64_t)a.b * a.h_kv * a.s_kv * D;
      const int64_t off = (int64_t)sp * plane + (((int64_t)bi * a.h_kv + g) * a.s_kv + my_key) * D;
      float* pk = part + off;
      float* pv = part + (int64_t)n_split * plane + off;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d0 = db * 32 + 8 * rq + 4 * h;
          *(f32x4*)(pk + d0) = f32x4{dk[db][4 * rq] * a.dk_scale, dk[db][4 * rq + 1] * a.dk_scale,
                                     dk[db][4 * rq + 2] * a.dk_scale, dk[db][4 * rq + 3] * a.dk_scale};
          *(f32x4*)(pv + d0) =
              f32x4{dv[db][4 * rq] * vsc, dv[db][4 * rq + 1] * vsc, dv[db][4 * rq + 2] * vsc, dv[db][4 * rq + 3] * vsc};
        }
    }
  };
  store_keys(dk0, dv0, key0);
  store_keys(dk1, dv1, key1);
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
// Pipelined like the forward: the K/V tile of step t+2 is loaded into
// registers while step t is computed and written to the other LDS buffer at
// step t+1. K and V tiles are row-major in the bswz layout; the K^T operand of
// dQ^T += K^T dS^T comes from the same K tile through ds_read_b64_tr_b16.
template <typename T, int D, bool CAUSAL, int MOD>
__global__ __launch_bounds__(64 * dq_waves(D), 8 / dq_waves(D)) void bwd_dq_kernel(BwdArgs a, int n_qblk) {
  typedef typename T::vec8 V8;
  constexpr int kQBlock = 32 * dq_waves(D);
  typedef BswzTile<kKTile, D, 64 * dq_waves(D)> KvTile;
  constexpr int NKS = D / 16, NDB = D / 32, NSB = kKTile / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKTile * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kKTile * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int bh_total = a.b * a.h_q;
  const int rank = blockIdx.x / bh_total;
  const int slot = xcd_slot(blockIdx.x - rank * bh_total, bh_total, a.h_q / a.h_kv);  // KV group: one XCD
  const int qb = n_qblk - 1 - rank;
  const int bi = slot / a.h_q, hq = slot - (slot / a.h_q) * a.h_q;
  const int g = hq / (a.h_q / a.h_kv);
  const int qblk0 = qb * kQBlock;
  const int q0 = qblk0 + wave * 32;
  const int my_q = q0 + j;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const uint16_t* qp = (const uint16_t*)a.q + bi * a.qs.b + hq * a.qs.h;
  const uint16_t* dop = (const uint16_t*)a.dout + bi * a.dos.b + hq * a.dos.h;
  const uint16_t* kp = (const uint16_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint16_t* vp = (const uint16_t*)a.v + bi * a.vs.b + g * a.vs.h;

  V8 qf[NKS], df[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    if (my_q < L.lq) {
      qf[t] = *(const V8*)(qp + (int64_t)my_q * a.qs.s + 16 * t + 8 * h);
      df[t] = *(const V8*)(dop + (int64_t)my_q * a.dos.s + 16 * t + 8 * h);
    } else {
      qf[t] = V8{};
      df[t] = V8{};
    }
  }
  const int64_t row_bh = ((int64_t)bi * a.h_q + hq) * a.s_q;
  // Rows past lq have Q = dO = 0, so their dS and dQ are 0. A row that sees
  // no key has LSE = -inf and every score masked: 0 keeps its P at 0.
  const float lse = my_q < L.lq ? a.lse[row_bh + my_q] : 0.f;
  const float lse2 = lse == -INFINITY ? 0.f : lse * kLog2e;
  // D = rowsum(dO * O) of this row: this lane holds half of the row's dO
  // (elements 16 t + 8 h .. +7) and reads the same half of O; the halves are
  // summed across the wave. The dK/dV kernel, launched next, reads D from the
  // workspace (rows past lq hold 0 and are never used).
  float dpart = 0.f;
  if (my_q < L.lq) {
    const uint16_t* op = (const uint16_t*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)my_q * a.os.s;
#pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const u32x4 ov = *(const u32x4*)(op + 16 * t + 8 * h);
      const u32x4 dv = __builtin_bit_cast(u32x4, df[t]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dpart = fmaf(to_f32<T>((uint16_t)(ov[w] & 0xffff)), to_f32<T>((uint16_t)(dv[w] & 0xffff)), dpart);
        dpart = fmaf(to_f32<T>((uint16_t)(ov[w] >> 16)), to_f32<T>((uint16_t)(dv[w] >> 16)), dpart);
      }
    }
  }
  const float dl = wave_sum_halves(dpart) * a.delta_scale;
  if (h == 0 && my_q < a.s_q) a.delta[row_bh + my_q] = dl;
  const float slope2 = (MOD && a.mod.slopes != nullptr) ? a.mod.slopes[hq] * kLog2e : 0.f;
  const void* bias_row =
      (MOD == kModAll && a.mod.bias != nullptr && my_q < a.s_q)
          ? (const void*)((const char*)a.mod.bias +
                          (bi * a.mod.bb + hq * a.mod.bh + (int64_t)my_q * a.mod.bs) * (a.mod.bias_f32 ? 4 : 2))
          : nullptr;
  const float sl2 = a.scale * kLog2e;

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

  // This lane's row-operand offsets in a K / V tile: row j (+ 32 nb), chunk 2 t + h.
  int rowoff[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) rowoff[t] = j * D + (((2 * t + h) ^ bswz<D>(j)) * 8);
  TrLaneB<D> trl;
  trl.init(lane);

  const int kv_end = qblk0 >= L.lq ? 0 : CAUSAL ? max(0, min(L.lk, min(qblk0 + kQBlock, L.lq) + L.off)) : L.lk;
  const int n_tiles = (kv_end + kKTile - 1) / kKTile;
  KvTile kreg, vreg;
  kreg.init(a.ks.s, tid);
  vreg.init(a.vs.s, tid);
  // Bytes a tile may read: all its rows, or up to key lk - 1 in the last
  // tile (keys at or past lk read as zero); none past the last tile, so the
  // loads issued there read nothing and need no branch.
  const uint32_t kfull = tile_bytes(0, kKTile, a.ks.s, D, 2), vfull = tile_bytes(0, kKTile, a.vs.s, D, 2);
  const uint32_t klast = tile_bytes((n_tiles - 1) * kKTile, L.lk, a.ks.s, D, 2);
  const uint32_t vlast = tile_bytes((n_tiles - 1) * kKTile, L.lk, a.vs.s, D, 2);
  auto load_tile = [&](int tile) {
    const bool last = tile == n_tiles - 1, none = tile >= n_tiles;
    kreg.load(kp, tile * kKTile, none ? 0u : last ? klast : kfull);
    vreg.load(vp, tile * kKTile, none ? 0u : last ? vlast : vfull);
  };
  auto store_tile = [&](int buf) {
    kreg.store(Ks[buf]);
    vreg.store(Vs[buf]);
  };
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    load_tile(1);
  }
  // One K/V tile. Unrolled by two, `buf` is a constant at each call, so every
  // LDS operand address is a per-lane offset plus an immediate instead of an
  // offset combined with a run-time buffer base. The other buffer is written
  // every step (past the last tile with zeros nobody reads).
  auto step = [&](const int tile, const int buf) {
    const int k0 = tile * kKTile;
    __syncthreads();  // buffer `buf` is complete; buffer buf^1 is no longer read
    store_tile(buf ^ 1);
    load_tile(tile + 2);
    if (CAUSAL && k0 > q0 + 31 + L.off) return;  // every key of the tile is above this wave's rows
    f32x16 s[NSB], dp[NSB];
#pragma unroll
    for (int nb = 0; nb < NSB; ++nb) {
      s[nb] = f32x16{};
      dp[nb] = f32x16{};
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const V8 ka = *(const V8*)(&Ks[buf][nb * 32 * D + rowoff[t]]);
        s[nb] = T::mfma(ka, qf[t], s[nb]);
        const V8 va = *(const V8*)(&Vs[buf][nb * 32 * D + rowoff[t]]);
        dp[nb] = T::mfma(va, df[t], dp[nb]);
      }
    }
    if constexpr (MOD == kModNone) {
      // Operand reads issued kLookQ MFMAs ahead of their MFMA.
      constexpr int kLookQ = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, kLookQ, 0);
#pragma unroll
      for (int i = 0; i < 2 * NSB * NKS - kLookQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kLookQ, 0);
    }
    const bool need_mask = (k0 + kKTile > L.lk) || (CAUSAL && k0 + kKTile - 1 > q0 + L.off);
    if (need_mask) {
      // Key k0 + c (c = 32 nb + acc_row(r, h)) is hidden from this row iff it
      // is past the row's last visible key: one compare against a constant.
      const int lim = (CAUSAL ? min(L.lk - 1, my_q + L.off) : L.lk - 1) - k0 - 4 * h;
#pragma unroll
      for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (nb * 32 + acc_row(r, 0) > lim) s[nb][r] = -INFINITY;
    }
    // Score modifiers of this query row and the tile's keys, log2 units.
    float madd[NSB][16];
#pragma unroll
    for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) madd[nb][r] = 0.f;
    if (MOD) {
#pragma unroll
      for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int key0 = k0 + nb * 32 + 8 * q4 + 4 * h;
          const f32x4 bv = MOD == kModAll ? bias4<T>(bias_row, a.mod.bias_f32, key0, a.s_kv) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            madd[nb][4 * q4 + e] = fmaf(bv[e], kLog2e, -slope2 * fabsf((float)(my_q + L.off - (key0 + e))));
        }
    }
    uint32_t dspk[NSB][8];
#pragma unroll
    for (int nb = 0; nb < NSB; ++nb) {
      // Dropout words of this row for the key groups q4 = 0..3: the four lanes
      // of a query quad draw one block each (q4 = lane & 3) and trade words.
      u32x4 dw = u32x4{0u, 0u, 0u, 0u};
      if (MOD >= kModDrop && a.mod.drop_k8 < 256) {
        const u32x4 w = drop_words((uint32_t)(k0 + nb * 32 + 8 * (lane & 3) + 4 * h) >> 2, (uint32_t)my_q >> 2,
                                   (uint32_t)(bi * a.h_q + hq), a.mod.offset, a.mod.seed_lo, a.mod.seed_hi);
        dw = quad_transpose(w, lane);
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[nb][r], sl2, madd[nb][r] - lse2));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[nb][r + 1], sl2, madd[nb][r + 1] - lse2));
        float z0 = 1.f, z1 = 1.f;  // dS = P (Z dP - D)
        if (MOD >= kModDrop) {
          z0 = drop_keep(dw[r / 4], r % 4, a.mod.drop_k8) ? a.mod.drop_scale : 0.f;
          z1 = drop_keep(dw[r / 4], (r + 1) % 4, a.mod.drop_k8) ? a.mod.drop_scale : 0.f;
        }
        dspk[nb][r / 2] = pack2<T>(p0 * (z0 * dp[nb][r] - dl), p1 * (z1 * dp[nb][r + 1] - dl));
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t2 = 0; t2 < kKTile / 16; ++t2) {
      const int nb = t2 / 2, base = 4 * (t2 % 2);
      const V8 sb = __builtin_bit_cast(
          V8, u32x4{dspk[nb][base], dspk[nb][base + 1], dspk[nb][base + 2], dspk[nb][base + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = T::mfma(trl.template tr<V8>(Ks[buf], db, t2), sb, dq[db]);
    }
    if constexpr (MOD == kModNone) {  // the same for the K^T reads, two per MFMA
      constexpr int kLookQ = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLookQ, 1);
#pragma unroll
      for (int i = 0; i < (kKTile / 16) * NDB - kLookQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kLookQ, 1);
    }
  };
  if constexpr (MOD == kModAll) {  // (the bias loads' registers leave no room for two copies)
    for (int tile = 0; tile < n_tiles; ++tile) step(tile, tile & 1);
  } else {
    for (int tile = 0; tile < n_tiles; tile += 2) {
      step(tile, 0);
      if (tile + 1 < n_tiles) step(tile + 1, 1);
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
        w.x = pack2<T>(dq[db][4 * rq] * a.dq_scale, dq[db][4 * rq + 1] * a.dq_scale);
        w.y = pack2<T>(dq[db][4 * rq + 2] * a.dq_scale, dq[db][4 * rq + 3] * a.dq_scale);
        *(u32x2*)(dqp + d0) = w;
      }
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T, int D, int MOD>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream, const TimingEvents& te) {
  const bool timed = te.n >= 3;
  // dQ first: it also writes D = rowsum(dO * O), which dK/dV reads.
  if (timed) (void)hipEventRecord(te.ev[0], stream);
  const int n_qblk = (a.s_q + 32 * dq_waves(D) - 1) / (32 * dq_waves(D));
  const dim3 g2(n_qblk * a.b * a.h_q);
  if (a.causal)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, true, MOD>), g2, dim3(64 * dq_waves(D)), 0, stream, a, n_qblk);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, false, MOD>), g2, dim3(64 * dq_waves(D)), 0, stream, a, n_qblk);
  if (timed) (void)hipEventRecord(te.ev[1], stream);

  const int n_split = bwd_split_count(a.b, a.h_q, a.h_kv, a.s_kv, kKvBlock);
  float* part = n_split > 1 ? bwd_partials(a) : nullptr;
  const int n_kblk = (a.s_kv + kKvBlock - 1) / kKvBlock;
  const dim3 g1(n_kblk * a.b * a.h_kv * n_split);
  if (D == 128 && MOD == kModNone) {
    if (a.causal)
      hipLaunchKernelGGL((bwd_dkdv64_kernel<T, true>), g1, dim3(256), 0, stream, a, n_split, part);
    else
      hipLaunchKernelGGL((bwd_dkdv64_kernel<T, false>), g1, dim3(256), 0, stream, a, n_split, part);
  } else if (a.causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true, MOD>), g1, dim3(512), 0, stream, a, n_kblk, n_split, part);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false, MOD>), g1, dim3(512), 0, stream, a, n_kblk, n_split, part);
  if (n_split > 1) {
    const int64_t n4 = (int64_t)a.b * a.h_kv * a.s_kv * D / 4 * 2;
    const int64_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                       stream, a, n_split, (const float*)part);
  }
  if (timed) (void)hipEventRecord(te.ev[2], stream);
  return hipGetLastError();
}

}  // namespace

// Number of workgroups a KV head's query-head group is split over: enough
// to put at least 512 dK/dV workgroups in flight when the group allows it.
// The workspace is sized for the 256-key blocks of the 16-bit kernels; fewer
// keys per workgroup give more workgroups, hence never a larger split.
int bwd_split_count(int b, int h_q, int h_kv, int s_kv, int keys_per_wg) {
  const int G = h_q / h_kv;
  const int64_t base = (int64_t)((s_kv + keys_per_wg - 1) / keys_per_wg) * b * h_kv;
  int n = 1;
  while (base * n < 512 && 2 * n <= G && G % (2 * n) == 0) n *= 2;
  return n;
}

float* bwd_partials(const BwdArgs& a) {
  const int64_t rows = (int64_t)a.b * a.h_q * a.s_q;
  return (float*)((char*)a.delta + align256((size_t)rows * sizeof(float)));
}

hipError_t launch_bwd_reduce(const BwdArgs& a, int n_split, const float* part, hipStream_t stream) {
  const int64_t n4 = (int64_t)a.b * a.h_kv * a.s_kv * a.d / 4 * 2;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL((bwd_reduce_kernel<Bf16T>), dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                     stream, a, n_split, part);
  return hipGetLastError();
}

size_t bwd_workspace_bytes(int b, int h_q, int h_kv, int s_q, int s_kv, int d) {
  size_t bytes = align256((size_t)b * h_q * s_q * sizeof(float));
  const int n_split = bwd_split_count(b, h_q, h_kv, s_kv, kKvBlock);
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

template <int MOD>
hipError_t launch_bwd_m(const BwdArgs& a, Io io, hipStream_t stream, const TimingEvents& te) {
  if (io == Io::BF16)
    return a.d == 64 ? launch_all<Bf16T, 64, MOD>(a, stream, te) : launch_all<Bf16T, 128, MOD>(a, stream, te);
  return a.d == 64 ? launch_all<F16T, 64, MOD>(a, stream, te) : launch_all<F16T, 128, MOD>(a, stream, te);
}

hipError_t launch_bwd(const BwdArgs& a, Io io, hipStream_t stream, const TimingEvents& te) {
  switch (mod_level(a.mod)) {
    case kModAll: return launch_bwd_m<kModAll>(a, io, stream, te);
    case kModDrop: return launch_bwd_m<kModDrop>(a, io, stream, te);
    case kModAlibi: return launch_bwd_m<kModAlibi>(a, io, stream, te);
    default: return launch_bwd_m<kModNone>(a, io, stream, te);
  }
}

}  // namespace sdpa
