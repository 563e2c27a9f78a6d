// FP8 (e4m3) forward: fused attention with fp8 inputs, fp32 accumulation and
// bf16 output.
//
// What is computed: the same attention as the 16-bit forward (JAX attention
// codelab, step 1 formula; cuDNN 9 blog, "SDPA as a cuDNN graph", Figure 4),
// on inputs given as OCP e4m3 codes with per-tensor fp32 descale factors
// (codelab step 10: E4M3 in the forward pass, per-tensor scaling recipe):
//   Q = q8 * descale_q,  K = k8 * descale_k,  V = v8 * descale_v,
//   S = attn_scale * Q K^T (masked), P = softmax(S), O = P V, LSE.
// The fp8 forward on H200 is the cuDNN 9 blog's 1.2 PFLOPS figure (head dim
// 256, no causal mask).
//
// Arithmetic: S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 with the
// raw codes (exact products, fp32 sum); attn_scale * descale_q * descale_k is
// folded into the exp2 argument. The softmax weights p = exp(S - m) <= 1 are
// quantised to e4m3 as p * scale_p for the second matmul O^T += V^T P^T (also
// fp8 MFMA); the row sum l uses the unquantised fp32 p. O = O_acc * descale_v *
// descale_p / l. The running max is kept exact (every increase rescales), so
// p <= 1, p * scale_p never exceeds the e4m3 range when scale_p <= 448, and
// the largest weight of a row is exactly scale_p: a running max that trails
// the row max leaves that weight to e4m3 rounding (3 mantissa bits), which
// on a row dominated by one late key moved O by up to 0.14.
//
// Layout: one workgroup = 4 waves x 32 query rows at d = 128, 8 at d = 256;
// each lane owns one query column of S^T. K and V tiles (64 keys) are staged
// row-major in LDS (V with swizzled 16-byte chunks); the V^T operand of the
// second matmul is read with ds_read_b64_tr_b8, each lane's 32 keys in the
// order of the accumulator registers the P operand is packed from. (Staging V
// transposed through registers took 32 byte permutes per tile on the staging
// threads: the transposed reads are 0.360 -> 0.332 ms at d = 128 causal
// s8192 and 1.008 -> 0.987 ms at d = 256, same-box A/B.)
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Waves (of 32 query rows) per workgroup: 8 at d = 256 (one workgroup per
// CU, one K/V staging for eight waves), 4 at d = 128 (three per CU).
constexpr int fp8_waves(int d) { return d == 256 ? 8 : 4; }
constexpr int kBN8 = 64;     // keys per tile (one 64-deep MFMA step of P V)

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = e4m3 for both operands, unit E8M0 scales (127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ds_read_b64_tr_b8: within each 16-lane group, lane i receives byte i % 8
// of the 8-byte pieces addressed by lanes 2 k + i / 8 of the group, k = 0..7
// (byte k of the result from piece k).
__device__ __forceinline__ u32x2 ds_read_tr8(const uint8_t* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p)));
}

// Chunk swizzle of the row-major V tile (16-byte chunks): row r keeps chunk c
// at position c ^ vswz8(r). The transposed reads of one pass (32 lanes) take a
// 32-byte column segment of the 8 rows 16 u + {0..3, 8..11} (+4 in the other
// half-wave); with 128- or 256-byte rows, rows of equal parity would share
// banks, and the XOR (bits 1 and 3 of the row -> chunk bits 1 and 2) moves
// the four rows of each parity to four different 32-byte bank groups.
// Invariant under +16 rows.
__device__ __forceinline__ int vswz8(int r) { return (((r >> 1) & 1) | ((r >> 2) & 2)) << 1; }

template <int D, bool CAUSAL>
// Occupancy: at d = 256 one 8-wave workgroup per CU (about 245 VGPRs, 66 KB
// LDS), at d = 128 three 4-wave workgroups (about 165 VGPRs, 34 KB LDS each):
// a second (third) wave per
// SIMD hides the softmax VALU work behind the other waves' MFMAs. At d = 256
// the 8 waves share one K/V staging, which also halves each thread's staging
// registers: two 4-wave workgroups per CU spilled 10 VGPRs and took 1.27 ms
// on b4 h8 s8192, the 8-wave form 1.15 ms (same-box A/B; one wave per SIMD:
// 2.28 ms). At d = 128, 8 waves (two per SIMD) lose to three 4-wave
// workgroups: 0.44 vs 0.40 ms on b2 h16 s8192 causal.
__global__ __launch_bounds__(64 * fp8_waves(D), D == 256 ? 1 : 3) void fwd_fp8_kernel(FwdArgs a, int n_qblk) {
  constexpr int kNW = fp8_waves(D);
  constexpr int kBM8 = 32 * kNW;
  constexpr int NT = 64 * kNW;
  constexpr int KSTR = D + 16;       // bytes per K row in LDS
  constexpr int VCPR = D / 16;       // 16-byte chunks per V row
  constexpr int NKS = D / 64;        // 64-deep contraction steps over d
  constexpr int NDB = D / 32;        // 32-wide output blocks over d
  constexpr int KCH = kBN8 * D / 16 / NT;   // 16-byte K chunks per thread
  static_assert(KCH >= 1 && KCH * NT * 16 == kBN8 * D, "tile map");
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][kBN8 * KSTR];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2][kBN8 * D];  // row-major, vswz8 chunks

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int bh_total = a.b * a.h_q;
  const int rank = blockIdx.x / bh_total;
  const int slot = xcd_slot(blockIdx.x - rank * bh_total, bh_total, a.h_q / a.h_kv);  // KV group: one XCD
  const int qb = n_qblk - 1 - rank;
  const int bi = slot / a.h_q, hq = slot - (slot / a.h_q) * a.h_q;
  const int g = hq / (a.h_q / a.h_kv);
  const int qblk0 = qb * kBM8;
  const int q0 = qblk0 + wave * 32;
  const int my_q = q0 + j;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const uint8_t* qp = (const uint8_t*)a.q + bi * a.qs.b + hq * a.qs.h;
  const uint8_t* kp = (const uint8_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint8_t* vp = (const uint8_t*)a.v + bi * a.vs.b + g * a.vs.h;

  // Q row bytes 64 t + 32 h .. +31 of this lane's query (B operand of S^T).
  i32x8 qf[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    if (my_q < L.lq) {
      const u32x4 lo = *(const u32x4*)(qp + (int64_t)my_q * a.qs.s + 64 * t + 32 * h);
      const u32x4 hi = *(const u32x4*)(qp + (int64_t)my_q * a.qs.s + 64 * t + 32 * h + 16);
      qf[t] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      qf[t] = i32x8{};
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const float lsp = __log2f(a.scale_p);  // weights are produced pre-multiplied by scale_p

  const int kv_end = qblk0 >= L.lq ? 0 : CAUSAL ? max(0, min(L.lk, min(qblk0 + kBM8, L.lq) + L.off)) : L.lk;
  const int n_tiles = (kv_end + kBN8 - 1) / kBN8;

  // Staging map. K: 16-byte chunks (row r, chunk cc).
  constexpr int KCPR = D / 16;  // K chunks per row
  uint32_t koff[KCH], kdst[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = tid + NT * i;
    const int r = c / KCPR, cc = c % KCPR;
    koff[i] = (uint32_t)(r * a.ks.s + cc * 16);
    kdst[i] = r * KSTR + cc * 16;
  }
  // V: 16-byte chunks like K, written row-major in the vswz8 layout.
  uint32_t voff[KCH], vdst[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = tid + NT * i;
    const int r = c / VCPR, cc = c % VCPR;
    voff[i] = (uint32_t)(r * a.vs.s + cc * 16);
    vdst[i] = r * D + ((cc ^ vswz8(r)) * 16);
  }
  u32x4 kreg[KCH];
  u32x4 vreg[KCH];
  auto load_tile = [&](int k0) {
    // Rows at or past lk read as zero (never the caller's padding).
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + (int64_t)k0 * a.ks.s, tile_bytes(k0, L.lk, a.ks.s, D, 1));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + (int64_t)k0 * a.vs.s, tile_bytes(k0, L.lk, a.vs.s, D, 1));
#pragma unroll
    for (int i = 0; i < KCH; ++i) kreg[i] = buf_load16(kr, koff[i]);
#pragma unroll
    for (int i = 0; i < KCH; ++i) vreg[i] = buf_load16(vr, voff[i]);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) *(u32x4*)(&Ks[buf][kdst[i]]) = kreg[i];
#pragma unroll
    for (int i = 0; i < KCH; ++i) *(u32x4*)(&Vs[buf][vdst[i]]) = vreg[i];
  };

  // Lane offsets of the transposed V reads. The A operand of O^T += V^T P^T
  // for output block db: lane (d row j, half h) holds the 32 keys whose P
  // bytes it meets, byte m = key 16 (m / 8) + 8 ((m % 8) / 4) + 4 h + m % 4
  // (the order P is packed in), as four ds_read_b64_tr_b8, read u giving bytes
  // 8 u .. 8 u + 7. For that, lane l of 16-lane group G addresses the 8-byte
  // piece of key row 16 u + 8 (k / 4) + 4 (G / 2) + k % 4, k = (l % 16) / 2, at
  // columns 32 db + 16 (G % 2) + 8 (l % 2): the row is one base plus 16 u rows.
  // (vswz8 only touches chunk bits 1-2, so blocks db and db + 4 of d = 256
  // are 128 bytes apart.)
  int vtr[4];
  {
    const int G = lane >> 4, L = lane & 15, k = L >> 1;
    const int r0 = 8 * (k >> 2) + 4 * (G >> 1) + (k & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) vtr[db] = r0 * D + (((2 * db + (G & 1)) ^ vswz8(r0)) * 16) + 8 * (L & 1);
  }

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    if (n_tiles > 1) load_tile(kBN8);
  }
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int k0 = tile * kBN8;
    const int buf = tile & 1;
    __syncthreads();
    if (tile + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (tile + 2 < n_tiles) load_tile((tile + 2) * kBN8);
    }

    // S^T = K Q^T (codes), two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sacc[nb] = f32x16{};
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const uint8_t* kr = &Ks[buf][(nb * 32 + j) * KSTR + 64 * t + 32 * h];
        const u32x4 lo = *(const u32x4*)kr, hi = *(const u32x4*)(kr + 16);
        const i32x8 kf = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sacc[nb] = mfma_fp8(kf, qf[t], sacc[nb]);
      }
    }
    const bool need_mask = (k0 + kBN8 > L.lk) || (CAUSAL && k0 + kBN8 - 1 > q0 + L.off);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + nb * 32 + acc_row(r, h);
          if (key >= L.lk || (CAUSAL && key > my_q + L.off)) sacc[nb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
    mx = wave_max_halves(mx) * sl2;
    if (__any(mx > m_run)) {
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
    // p * scale_p = exp2(S * scale * log2e - m + log2(scale_p)) in fp32: its
    // sum is l * scale_p; its e4m3 rounding is packed as the B operand, byte
    // m = 16 nb + r of this lane half.
    const float off = lsp - (m_run == -INFINITY ? 0.f : m_run);  // all -inf scores: P = 0
    uint32_t pw[8];
    float ls0, ls1;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int nb = w >> 2, r = 4 * (w & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r], sl2, off));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r + 1], sl2, off));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r + 2], sl2, off));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[nb][r + 3], sl2, off));
      ls0 = w == 0 ? p0 + p2 : ls0 + (p0 + p2);
      ls1 = w == 0 ? p1 + p3 : ls1 + (p1 + p3);
      // The low-half convert keeps the old upper 16 bits, which the high-half
      // convert then overwrites: any register serves as the old value (p0's
      // bits here), so no zero has to be materialised first.
      uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, (int)__builtin_bit_cast(uint32_t, p0), false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pw[w] = word;
    }
    l_run += ls0 + ls1;
    const i32x8 pb = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    // O^T += V^T P^T over the 64 keys of the tile.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint8_t* vr = &Vs[buf][vtr[db & 3] + 128 * (db >> 2)];
      const u32x2 r0 = ds_read_tr8(vr), r1 = ds_read_tr8(vr + 16 * D), r2 = ds_read_tr8(vr + 32 * D),
                  r3 = ds_read_tr8(vr + 48 * D);
      const i32x8 va = i32x8{(int)r0.x, (int)r0.y, (int)r1.x, (int)r1.y, (int)r2.x, (int)r2.y, (int)r3.x, (int)r3.y};
      oacc[db] = mfma_fp8(va, pb, oacc[db]);
    }
  }

  const float l_tot = wave_sum_halves(l_run);  // = l * scale_p
  // Rows past lq, and rows that see no key: O = 0, LSE = -inf.
  const bool live = my_q < L.lq && l_tot > 0.f;
  const float inv = live ? a.descale_v * a.descale_p * a.scale_p / l_tot : 0.f;
  if (my_q < a.s_q) {
    uint16_t* op = (uint16_t*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)my_q * a.os.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 w;
        w.x = pack2<Bf16T>(oacc[db][4 * rq + 0] * inv, oacc[db][4 * rq + 1] * inv);
        w.y = pack2<Bf16T>(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv);
        *(u32x2*)(op + d0) = w;
      }
    if (a.lse != nullptr && h == 0)
      a.lse[((int64_t)bi * a.h_q + hq) * a.s_q + my_q] = live ? (m_run + __log2f(l_tot) - lsp) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const int bm = 32 * fp8_waves(D);
  const int n_qblk = (a.s_q + bm - 1) / bm;
  const dim3 grid(n_qblk * a.b * a.h_q), block(64 * fp8_waves(D));
  if (a.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, true>), grid, block, 0, stream, a, n_qblk);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), grid, block, 0, stream, a, n_qblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_d<128>(a, stream) : launch_d<256>(a, stream);
}

}  // namespace sdpa
