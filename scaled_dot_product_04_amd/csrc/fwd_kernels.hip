// Forward kernels: fused scaled dot-product attention with online softmax.
//
// What is computed (JAX attention codelab, step 1 formula and step 7 causal
// mask; cuDNN 9 blog, "SDPA as a cuDNN graph", Figure 4: the scale multiplies
// the first matmul's output, the causal mask is an index compare + select,
// softmax follows, then the second matmul; the node's second output "stats"
// is the per-row logsumexp):
//   S = scale * Q K^T, masked (j > i) under the causal flag, O = softmax(S) V,
//   LSE_i = ln sum_j exp(S_ij).
// The score matrix is never written to memory: each workgroup streams K/V
// tiles through LDS and keeps a running row max m and row sum l (the flash
// attention recurrence the cuDNN blog's "SDPA performance" section cites).
//
// gfx950 design (d = 128: one workgroup = 8 waves = 256 query rows of one
// (b, head), or 4 waves = 128 rows for up to 1024 keys; d = 64: 4 waves):
//  * each wave owns 32 query rows; it holds its Q rows in registers as the
//    B operand of S^T = K Q^T (v_mfma_f32_32x32x16), so every lane owns one
//    query column of S^T: the row max / row sum of the softmax are in-lane
//    reductions plus one exchange between the two wave halves;
//  * the exponentiated scores, packed to 16 bits, are directly the B operand
//    of O^T += V^T P^T; the V^T operand is read from the row-major V tile
//    (16-byte chunks swizzled per row) with ds_read_b64_tr_b16;
//  * K/V tiles (128 keys for the 8-wave d = 128 kernel, else 64) are staged in
//    LDS once per workgroup through registers, double-buffered, and shared by
//    the waves; under the causal mask, tiles entirely above the diagonal are
//    never loaded, and diagonal tiles are masked element-wise;
//  * without score modifiers no per-tile row max is taken: the weights use
//    the running max as it stands (started at the row's key-0 score) and are
//    rescaled by a power of two only when a tile's weights outgrow 2^8; an
//    fp32 overflow sends the workgroup back over its rows on the exact path;
//  * workgroups are issued longest-first for the causal mask, and heads are
//    remapped so that all query blocks of a head (and the query heads of a
//    GQA group) run on the same XCD and share its L2.
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {


// Maps a linear workgroup id to (query block, b, head). Query blocks are
// issued from the last (longest under the causal mask) to the first; within a
// rank, the query heads of one KV group share an XCD (xcd_slot).
__device__ __forceinline__ void map_block(int id, int n_qblk, int bh_total, int h_q, int G, int& qb, int& bi,
                                          int& hq) {
  const int rank = id / bh_total;
  const int slot = xcd_slot(id - rank * bh_total, bh_total, G);
  qb = n_qblk - 1 - rank;
  bi = slot / h_q;
  hq = slot - bi * h_q;
}


// NW waves per workgroup, 32 query rows per wave. MOD: score modifiers added
// to the scaled scores (kModAlibi: ALiBi slopes only; kModDrop: dropout and
// ALiBi; kModAll: also a bias tensor). KS = 2 splits the keys of each staged
// tile between two groups of NW / 2 waves that own the same query rows (for
// grids too small to fill the GPU: it halves the chain of tiles that the
// longest workgroup walks); the groups merge their (m, l, O) at the end.
template <typename T, int D, bool CAUSAL, int NW, int MOD, int KS>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_mfma_kernel(FwdArgs a, int n_qblk) {
  typedef typename T::elem E;
  typedef typename T::vec8 V8;
  static_assert(KS == 1 || (KS == 2 && MOD == kModNone && NW == 8), "key split: 8 waves, no modifiers");
  constexpr int NT = 64 * NW;    // threads
  constexpr int RW = NW / KS;    // waves per key group, each with its own 32 query rows
  constexpr int BM = 32 * RW;    // query rows per workgroup
  // Keys per K/V tile: 128 at d = 128 (halves the per-tile barrier, row-max
  // reduction and loop overhead; 246 VGPRs, 135 KB LDS at 8 waves), 64 at
  // d = 64 (keeps three waves per SIMD) and with score modifiers (their
  // registers would not fit beside 128-key score tiles).
  constexpr int kBN = (KS == 2 || (D == 128 && MOD == kModNone && NW == 8)) ? 128 : 64;
  constexpr int GBN = kBN / KS;  // keys of the tile that one wave takes
  constexpr int KSTR = D + 8;    // LDS row stride (elements) of the K tile
  constexpr int kLook = 4;       // MFMAs by which operand reads run ahead
  constexpr int NKS = D / 16;    // 16-wide contraction steps over d
  constexpr int NDB = D / 32;    // 32-wide output blocks over d
  constexpr int NSB = GBN / 32;  // 32-key score blocks per tile and wave
  constexpr int CH = D / 8;                    // 16-byte chunks per K or V row
  constexpr int KCH = kBN * CH / NT;           // K (and V) chunks staged per thread
  static_assert(KCH * NT == kBN * CH, "tile / thread mismatch");
  // Two K/V buffers: tile t is computed from buffer t%2 while tile t+1 is written
  // into the other one; loads for tile t+2 are in flight in registers meanwhile.
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * KSTR];
  // V tile row-major (swizzled 16-byte chunks); V^T operands via transposed reads.
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int grp = wave / RW, rw = wave - grp * RW;  // key group, row wave
  const int kg = grp * GBN;                         // the group's keys in a tile
  int qb, bi, hq;
  map_block(blockIdx.x, n_qblk, a.b * a.h_q, a.h_q, a.h_q / a.h_kv, qb, bi, hq);
  const int g = hq / (a.h_q / a.h_kv);
  const int qblk0 = qb * BM;
  const int q0 = qblk0 + rw * 32;
  const int my_q = q0 + j;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const E* qp = (const E*)a.q + bi * a.qs.b + hq * a.qs.h;
  const E* kp = (const E*)a.k + bi * a.ks.b + g * a.ks.h;
  const E* vp = (const E*)a.v + bi * a.vs.b + g * a.vs.h;

  // Q rows as the B operand of S^T = K Q^T.
  V8 qf[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    if (my_q < L.lq) {
      qf[t] = *(const V8*)(qp + (int64_t)my_q * a.qs.s + 16 * t + 8 * h);
    } else {
      qf[t] = V8{};
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max, in log2 units of the scaled scores
  float l_run = 0.f;        // running sum (this lane half's keys only)
  const float sl2 = a.scale * kLog2e;
  // With modifiers the scores are scaled (and shifted) as soon as they are
  // computed, so the row max and the exponent use them as they are.
  const float sc = MOD ? 1.f : sl2;
  const float slope2 = (MOD && a.mod.slopes != nullptr) ? a.mod.slopes[hq] * kLog2e : 0.f;
  const uint32_t drop_slot = (uint32_t)(bi * a.h_q + hq);
  const void* bias_row =
      (MOD == kModAll && a.mod.bias != nullptr && my_q < a.s_q)
          ? (const void*)((const char*)a.mod.bias +
                          (bi * a.mod.bb + hq * a.mod.bh + (int64_t)my_q * a.mod.bs) * (a.mod.bias_f32 ? 4 : 2))
          : nullptr;

  // Keys visible to some row of this block: below lk and, under the causal
  // mask, at most (last valid row) + off.
  const int kv_end = qblk0 >= L.lq ? 0 : CAUSAL ? max(0, min(L.lk, min(qblk0 + BM, L.lq) + L.off)) : L.lk;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // Staging map: thread owns 16-byte chunks (row r, chunk cc) of K and of V;
  // consecutive threads read consecutive chunks of a row from HBM. K rows are
  // padded in LDS, V rows are swizzled. Chunk i of a thread is row
  // tid / CH + i * RS, chunk tid % CH: its LDS offset is the thread's base plus
  // a constant, its global offset the base plus i row strides (recomputed per
  // tile from an opaque copy, which keeps one register per tensor live
  // instead of KCH). Tiles move the buffer base.
  static_assert(NT % CH == 0, "whole rows per thread step");
  constexpr int RS = NT / CH;  // rows between a thread's chunks
  const int r0 = tid / CH, cc0 = tid % CH;
  const uint32_t koff0 = (uint32_t)(r0 * a.ks.s * 2 + cc0 * 16);
  const uint32_t voff0 = (uint32_t)(r0 * a.vs.s * 2 + cc0 * 16);
  const uint32_t kstep = (uint32_t)(RS * a.ks.s * 2), vstep = (uint32_t)(RS * a.vs.s * 2);
  // vswz depends on the row only through r % 4 (d = 128) or (r / 2) % 2
  // (d = 64), which RS (a multiple of 4) leaves unchanged.
  static_assert(RS % 4 == 0, "swizzle period");
  const int kdst0 = r0 * KSTR + cc0 * 8;
  const int vdst0 = r0 * D + ((cc0 ^ vswz<D>(r0)) * 8);
  auto kdst = [&](int i) { return kdst0 + i * RS * KSTR; };
  auto vdst = [&](int i) { return vdst0 + i * RS * D; };
  u32x4 vreg2[KCH];
  SwzLaneF<D> sl;
  sl.init(lane);
  u32x4 kreg[KCH];
  // Bytes a tile's descriptor allows: every row of a full tile, rows up to
  // lk - 1 in the last one (rows at or past lk read as zero, never the
  // caller's padding), none past the last tile (its loads read nothing).
  const uint32_t kfull = tile_bytes(0, kBN, a.ks.s, D, 2), vfull = tile_bytes(0, kBN, a.vs.s, D, 2);
  const uint32_t klast = tile_bytes((n_tiles - 1) * kBN, L.lk, a.ks.s, D, 2);
  const uint32_t vlast = tile_bytes((n_tiles - 1) * kBN, L.lk, a.vs.s, D, 2);
  auto load_tile = [&](int tile) {
    const int k0 = tile * kBN;
    const bool last = tile == n_tiles - 1, none = tile >= n_tiles;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + (int64_t)k0 * a.ks.s, none ? 0u : last ? klast : kfull);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + (int64_t)k0 * a.vs.s, none ? 0u : last ? vlast : vfull);
    uint32_t ko = koff0, vo = voff0;
    asm volatile("" : "+v"(ko), "+v"(vo));
#pragma unroll
    for (int i = 0; i < KCH; ++i) kreg[i] = buf_load16(kr, ko + i * kstep);
#pragma unroll
    for (int i = 0; i < KCH; ++i) vreg2[i] = buf_load16(vr, vo + i * vstep);
  };
  // Registers -> LDS buffer.
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) *(u32x4*)(&Ks[buf][kdst(i)]) = kreg[i];
#pragma unroll
    for (int i = 0; i < KCH; ++i) *(u32x4*)(&Vs[buf][vdst(i)]) = vreg2[i];
  };

  // The tile loop. fast (no modifiers only): the weights of a tile are taken
  // against the running max without its row max; returns true when a weight
  // overflowed, and the rows must be redone with fast = false.
  auto run = [&](const bool fast) -> bool {
    bool bad = false;
    if (n_tiles > 0) {
      load_tile(0);
      store_tile(0);
      load_tile(1);
    }

    for (int tile = 0; tile < n_tiles; ++tile) {
      const int k0 = tile * kBN;
      const int buf = tile & 1;
      __syncthreads();  // buffer `buf` is complete; buffer buf^1 is no longer read
      // Staging of tile + 1 (registers -> the other buffer) and the loads of
      // tile + 2: every thread takes part, every step (past the last tile the
      // stores write zeros nobody reads). A wave that computes the tile
      // stages after its score products, beside the exponentials, so the
      // scores start right after the barrier.
      auto stage = [&]() {
        store_tile(buf ^ 1);
        load_tile(tile + 2);
      };
      const int kg0 = k0 + kg;  // first key of this wave's part of the tile
      // Every key of it above this wave's rows: the wave only stages. (One
      // staging call site: with a second one in the skip branch the register
      // allocator kept two copies of the staging registers and spilled.)
      const bool skip = CAUSAL && kg0 > q0 + 31 + L.off;

      // S^T = K Q^T for this wave's GBN keys of the tile.
      f32x16 sacc[NSB];
      if (!skip) {
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb) {
          sacc[nb] = f32x16{};
#pragma unroll
          for (int t = 0; t < NKS; ++t) {
            const V8 kf = *(const V8*)(&Ks[buf][(kg + nb * 32 + j) * KSTR + 16 * t + 8 * h]);
            sacc[nb] = T::mfma(kf, qf[t], sacc[nb]);
          }
        }
        if constexpr (MOD == kModNone) {
          // Schedule: the K operand reads run kLook MFMAs ahead (the default
          // schedule read each operand just before its MFMA). 1.5 % on the hd128
          // forward, no extra spills.
          __builtin_amdgcn_sched_group_barrier(0x100, kLook, 0);  // LDS reads
#pragma unroll
          for (int i = 0; i < NSB * NKS - kLook; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kLook, 0);
        }
        if (MOD == kModNone && fast && tile == 0) {
          // Starting max: this row's score against the wave's first key kg
          // (unmasked; key 0 without a key split). A row's visible keys are a
          // prefix, so a row that sees any key this wave takes sees that one,
          // and an actual score is a lower bound of the row max: no weight
          // underflows for want of a larger one. (Rows that see none of the
          // wave's keys get no weight at all.) A row whose max is key 0, like
          // causal row 0, gets the weight exp2(0) = 1 for it, as with an exact
          // max. The first key is accumulator register 0 of the lower half-wave.
          m_run = halves_swap(sacc[0][0]).x * sc;  // lane j's value in both halves
        }
        if (MOD) {  // S * scale * log2e + (bias - slope * |i + off - j|) * log2e
#pragma unroll
          for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int key0 = kg0 + nb * 32 + 8 * q4 + 4 * h;
              const f32x4 bv = MOD == kModAll ? bias4<T>(bias_row, a.mod.bias_f32, key0, a.s_kv) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float dist = fabsf((float)(my_q + L.off - (key0 + e)));
                sacc[nb][4 * q4 + e] = fmaf(sacc[nb][4 * q4 + e], sl2, fmaf(bv[e], kLog2e, -slope2 * dist));
              }
            }
        }
        // Causal / key-length mask (only tiles that cross the diagonal or lk).
        const bool need_mask = (kg0 + GBN > L.lk) || (CAUSAL && kg0 + GBN - 1 > q0 + L.off);
        if (need_mask) {
          // Key k0 + c (c = nb * 32 + acc_row(r, h)) is visible iff k0 + c <= last,
          // the last key this row sees; one compare against a constant per score.
          const int last = CAUSAL ? min(L.lk - 1, my_q + L.off) : L.lk - 1;
          const int lim = last - kg0 - 4 * h;
#pragma unroll
          for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (nb * 32 + acc_row(r, 0) > lim) sacc[nb][r] = -INFINITY;
        }
      }
      stage();
      if (skip) continue;
      uint32_t pk[NSB][8];
      float lsum0 = 0.f, lsum1 = 0.f;
      if (MOD == kModNone && fast) {
        // Weights against the running max as it stands: no row max per tile.
        // The max only grows when a weight says so: every weight is >= 0, so
        // a lane sum <= 2^8 bounds each one by 2^8 (as the stale max of the
        // exact path does). Otherwise (rare) the lane's weights are scaled by
        // a power of two that brings their max into [1/2, 1), exactly, with O
        // and l; a weight that overflowed fp32 cannot be scaled, and the
        // workgroup redoes the rows on the exact path.
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            sacc[nb][r] = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r], sc, -m_run));
            sacc[nb][r + 1] = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r + 1], sc, -m_run));
            lsum0 += sacc[nb][r];
            lsum1 += sacc[nb][r + 1];
          }
        if (__any(!(lsum0 + lsum1 <= 256.f))) {
          float mx = 0.f;
#pragma unroll
          for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
          mx = wave_max_halves(mx);
          bad = bad || __any(!(mx <= 3.0e38f));
          const int e = mx > 1.f && mx <= 3.0e38f ? __builtin_amdgcn_frexp_expf(mx) : 0;
          m_run += (float)e;
          l_run = __builtin_amdgcn_ldexpf(l_run, -e);
          lsum0 = __builtin_amdgcn_ldexpf(lsum0, -e);
          lsum1 = __builtin_amdgcn_ldexpf(lsum1, -e);
#pragma unroll
          for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[nb][r] = __builtin_amdgcn_ldexpf(sacc[nb][r], -e);
#pragma unroll
          for (int i = 0; i < NDB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] = __builtin_amdgcn_ldexpf(oacc[i][r], -e);
        }
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) pk[nb][r / 2] = pack2<T>(sacc[nb][r], sacc[nb][r + 1]);
      } else {
        // Online softmax. The running max is only moved (and O, l rescaled) when
        // some row's max grew by more than 8 (log2 units): with a stale max the
        // weights stay below 2^8, and the final O / l and LSE are unchanged.
        float mx = -INFINITY;
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
        mx = wave_max_halves(mx) * sc;
        if (__any(mx > m_run + 8.f)) {
          const float m_new = fmaxf(m_run, mx);
          // A row that has seen no visible key yet keeps m = -inf (and O = l = 0).
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < NDB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        }

        // P = exp2(S * scale * log2e - m), packed to 16 bits as the B operand
        // (m = -inf only while every score of the row is -inf: P = 0).
        const float msub = m_run == -INFINITY ? 0.f : m_run;
        // Dropout words of this row for the tile's key groups (nb, q4): the four
        // lanes of a query quad draw one block each (q4 = lane & 3) and trade words.
        u32x4 dwq[NSB];
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb) {
          dwq[nb] = u32x4{0u, 0u, 0u, 0u};
          if (MOD >= kModDrop && a.mod.drop_k8 < 256) {
            const u32x4 w = drop_words((uint32_t)(kg0 + nb * 32 + 8 * (lane & 3) + 4 * h) >> 2, (uint32_t)my_q >> 2,
                                       drop_slot, a.mod.offset, a.mod.seed_lo, a.mod.seed_hi);
            dwq[nb] = quad_transpose(w, lane);
          }
        }
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r], sc, -msub));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r + 1], sc, -msub));
            lsum0 += p0;  // the row sum uses the undropped weights
            lsum1 += p1;
            if (MOD >= kModDrop) {
              // Dropout word of this row for the 4-key group of r (0, i.e. every
              // byte kept, without dropout); byte r % 4 decides key r.
              const uint32_t dw = dwq[nb][r / 4];
              const bool k_0 = drop_keep(dw, r % 4, a.mod.drop_k8);
              const bool k_1 = drop_keep(dw, (r + 1) % 4, a.mod.drop_k8);
              pk[nb][r / 2] = pack2<T>(k_0 ? p0 : 0.f, k_1 ? p1 : 0.f);
            } else {
              pk[nb][r / 2] = pack2<T>(p0, p1);
            }
          }
      }
      l_run += lsum0 + lsum1;

      // O^T += V^T P^T, 16 keys per step.
#pragma unroll
      for (int t2 = 0; t2 < GBN / 16; ++t2) {
        const int nb = t2 / 2, base = 4 * (t2 % 2);
        u32x4 bw = u32x4{pk[nb][base], pk[nb][base + 1], pk[nb][base + 2], pk[nb][base + 3]};
        const V8 pb = __builtin_bit_cast(V8, bw);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const V8 va = sl.template tr<V8>(Vs[buf] + kg * D, db, t2);
          oacc[db] = T::mfma(va, pb, oacc[db]);
        }
      }
      if constexpr (MOD == kModNone) {  // the same for the V^T reads, two per MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLook, 1);
#pragma unroll
        for (int i = 0; i < (GBN / 16) * NDB - kLook; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kLook, 1);
      }
    }
    return bad;
  };
  if constexpr (MOD == kModNone) {
    __shared__ int redo;
    if (tid == 0) redo = 0;  // the loop's barriers order this before any wave sets it
    if (run(true) && lane == 0) redo = 1;
    __syncthreads();
    if (redo) {  // (uniform over the workgroup)
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
      m_run = -INFINITY;
      l_run = 0.f;
      run(false);
    }
  } else {
    run(false);
  }
  if constexpr (KS == 2) {
    // Group 1 hands its running (O, m, l) to the group-0 wave with the same
    // rows through LDS (the K tile buffers, free once every wave is done):
    // m = max(m0, m1), O = O0 e^(m0 - m) + O1 e^(m1 - m), l likewise. A group
    // whose row total l is 0 saw no key of that row and adds nothing; its m
    // may be a masked key's score (the starting max), so it is left out of
    // the max too.
    constexpr int XS = NDB * 16 + 3;  // floats per lane
    static_assert(RW * 64 * XS * sizeof(float) <= sizeof(Ks), "merge buffer");
    float* const xp = reinterpret_cast<float*>(&Ks[0][0]) + (rw * 64 + lane) * XS;
    const float lt = wave_sum_halves(l_run);  // this group's row total
    __syncthreads();
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) xp[i * 16 + r] = oacc[i][r];
      xp[NDB * 16] = m_run;
      xp[NDB * 16 + 1] = l_run;
      xp[NDB * 16 + 2] = lt;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xp[NDB * 16], l1 = xp[NDB * 16 + 1], lt1 = xp[NDB * 16 + 2];
    const float m_new = fmaxf(lt == 0.f ? -INFINITY : m_run, lt1 == 0.f ? -INFINITY : m1);
    const float a0 = lt == 0.f ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float a1 = lt1 == 0.f ? 0.f : __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] = oacc[i][r] * a0 + xp[i * 16 + r] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = m_new;
  }

  // Epilogue: O = O_acc / l, LSE = ln l + m. Rows past lq, and rows that see
  // no key, get O = 0 and LSE = -inf.
  const float l_tot = wave_sum_halves(l_run);
  const bool live = my_q < L.lq && l_tot > 0.f;
  const float inv = live ? (MOD >= kModDrop ? a.mod.drop_scale : 1.f) / l_tot : 0.f;
  if (my_q < a.s_q) {
    E* op = (E*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)my_q * a.os.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 w;
        w.x = pack2<T>(oacc[db][4 * rq + 0] * inv, oacc[db][4 * rq + 1] * inv);
        w.y = pack2<T>(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv);
        *(u32x2*)(op + d0) = w;
      }
    if (a.lse != nullptr && h == 0)
      a.lse[((int64_t)bi * a.h_q + hq) * a.s_q + my_q] = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, int NW, int MOD, int KS = 1>
hipError_t launch_mfma_dm(const FwdArgs& a, hipStream_t stream) {
  const int bm = 32 * NW / KS;
  const int n_qblk = (a.s_q + bm - 1) / bm;
  const dim3 grid(n_qblk * a.b * a.h_q), block(64 * NW);
  if (a.causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, true, NW, MOD, KS>), grid, block, 0, stream, a, n_qblk);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, false, NW, MOD, KS>), grid, block, 0, stream, a, n_qblk);
  return hipGetLastError();
}

// The d = 64 forward splits each tile's keys between two wave groups when
// its 128-row blocks are too few to fill the GPU twice over and the rows are
// long enough for the chain of tiles to matter (the GPT-2-like b4 h12 s1024
// shape has 384 blocks of up to 16 tiles).
constexpr int kKeySplitMaxBlocks = 1024;
inline bool use_key_split(const FwdArgs& a) {
  const int64_t blocks = (int64_t)((a.s_q + 127) / 128) * a.b * a.h_q;
  return blocks <= kKeySplitMaxBlocks && a.s_kv >= 256;
}

template <typename T, int D, int NW>
hipError_t launch_mfma_d(const FwdArgs& a, hipStream_t stream) {
  switch (mod_level(a.mod)) {
    case kModAll: return launch_mfma_dm<T, D, NW, kModAll>(a, stream);
    case kModDrop: return launch_mfma_dm<T, D, NW, kModDrop>(a, stream);
    case kModAlibi: return launch_mfma_dm<T, D, NW, kModAlibi>(a, stream);
    default:
      if constexpr (D == 64) {
        if (use_key_split(a)) return launch_mfma_dm<T, D, 8, kModNone, 2>(a, stream);
      }
      return launch_mfma_dm<T, D, NW, kModNone>(a, stream);
  }
}

}  // namespace

// Up to 1024 keys the d = 128 forward runs 4-wave workgroups with 64-key tiles
// (two workgroups per CU, 67 KB LDS each): more of them in flight hides the
// prologue of these short blocks. Same-box sweep: s = 1024 0.130 -> 0.116 ms,
// s = 512 0.084 -> 0.080 ms; from s = 2048 on the 8-wave, 128-key kernel wins.
constexpr int kFwdSmallKeys = 1024;

hipError_t launch_fwd_mfma(const FwdArgs& a, Io io, hipStream_t stream) {
  const bool small = a.s_kv <= kFwdSmallKeys;
  if (io == Io::BF16) {
    if (a.d == 64) return launch_mfma_d<Bf16T, 64, 4>(a, stream);
    return small ? launch_mfma_d<Bf16T, 128, 4>(a, stream) : launch_mfma_d<Bf16T, 128, 8>(a, stream);
  }
  if (a.d == 64) return launch_mfma_d<F16T, 64, 4>(a, stream);
  return small ? launch_mfma_d<F16T, 128, 4>(a, stream) : launch_mfma_d<F16T, 128, 8>(a, stream);
}

}  // namespace sdpa
