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
// descale_p / l. The running max moves (and O, l are rescaled) only when a
// tile's row max exceeds it by more than kLazy8 (log2 units), so p <= 2^kLazy8;
// the weights are quantised as p * scale_p * 2^-kLazy8, which stays within the
// e4m3 range when scale_p <= 448. The factor cancels in O_acc / l, and the LSE
// adds it back.
//
// Layout: one workgroup = 4 waves x 32 query rows; each lane owns one query
// column of S^T. K tiles (64 keys) are staged row-major in LDS; V tiles are
// staged transposed, with the keys of each row permuted so that the 32 keys
// one lane half contributes to a 64-deep MFMA step are one contiguous 32-byte
// run (their order is the order of the accumulator registers the P operand
// is packed from).
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Waves (of 32 query rows) per workgroup: 8 at d = 256 (one workgroup per
// CU, one K/V staging for eight waves), 4 at d = 128 (three per CU).
constexpr int fp8_waves(int d) { return d == 256 ? 8 : 4; }
constexpr int kBN8 = 64;     // keys per tile (one 64-deep MFMA step of P V)
// Lazy running max: a row's max is only moved when it grows by more than this
// (log2 units). With an exact max, some row of a 32-row wave raises its max in
// most tiles of a long row, and each raise rescaled O (64 multiplies per lane):
// b2 h16 s8192 d128 causal 0.394 -> 0.363 ms, b4 h8 s8192 d256 1.118 -> 1.035
// ms (same-box A/B).
constexpr float kLazy8 = 2.f;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = e4m3 for both operands, unit E8M0 scales (127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Byte transpose of a 4x4 block: in[r] holds bytes (r, 0..3); out[c] holds
// bytes (0..3, c).
__device__ __forceinline__ void transpose4x4_b8(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

template <int D, bool CAUSAL>
// Occupancy: at d = 256 one 8-wave workgroup per CU (254 VGPRs, 74 KB LDS),
// at d = 128 three 4-wave workgroups (168 VGPRs): a second (third) wave per
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
  constexpr int VSTR = kBN8 + 16;    // bytes per transposed V row in LDS
  constexpr int NKS = D / 64;        // 64-deep contraction steps over d
  constexpr int NDB = D / 32;        // 32-wide output blocks over d
  constexpr int KCH = kBN8 * D / 16 / NT;   // 16-byte K chunks per thread
  constexpr int VTOT = kBN8 * D / 64;       // 4-key x 16-column V blocks per tile
  constexpr int VBL = (VTOT + NT - 1) / NT; // ... per thread
  static_assert(KCH >= 1 && KCH * NT * 16 == kBN8 * D && (VTOT % NT == 0 || VTOT < NT), "tile map");
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][kBN8 * KSTR];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[2][D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  // Staging map. K: 16-byte chunks (row r, chunk cc). V: blocks of 4 keys x 16
  // columns, loaded as four 16-byte row pieces and written transposed.
  constexpr int KCPR = D / 16;  // K chunks per row
  constexpr int VCG = D / 16;   // V column groups of 16
  uint32_t koff[KCH], kdst[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = tid + NT * i;
    const int r = c / KCPR, cc = c % KCPR;
    koff[i] = (uint32_t)(r * a.ks.s + cc * 16);
    kdst[i] = r * KSTR + cc * 16;
  }
  // At d = 256, block c is key group c % 16 of column group c / 16: the 64
  // lanes of one transposed store then write 16 different 4-byte positions
  // of only 4 rows (4 lanes per bank; with the column group fastest, the 16
  // lanes of a key group share a bank). Same-box A/B, b4 h8 s8192: 1.85 ->
  // 1.27 ms. At d = 128 the column group stays fastest: there the wider
  // row-contiguous global loads of that order matter more (0.41 vs 0.42 ms).
  uint32_t voff[VBL], vdst[VBL];
#pragma unroll
  for (int i = 0; i < VBL; ++i) {
    const int c = tid + NT * i;
    const int kg = D == 256 ? c % 16 : c / VCG;  // 4-key group 0..15
    const int cg = D == 256 ? c / 16 : c % VCG;
    voff[i] = (uint32_t)((4 * kg) * a.vs.s + 16 * cg);
    // key 4 kg = 32 blk + 8 gq + 4 hh  ->  position 32 hh + 16 blk + 4 gq
    const int blk = kg >> 3, gq = (kg & 7) >> 1, hh = kg & 1;
    vdst[i] = (16 * cg) * VSTR + 32 * hh + 16 * blk + 4 * gq;
  }
  u32x4 kreg[KCH];
  u32x4 vreg[VBL][4];
  const uint32_t vrow = (uint32_t)a.vs.s;
  auto load_tile = [&](int k0) {
    // Rows at or past lk read as zero (never the caller's padding).
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + (int64_t)k0 * a.ks.s, tile_bytes(k0, L.lk, a.ks.s, D, 1));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + (int64_t)k0 * a.vs.s, tile_bytes(k0, L.lk, a.vs.s, D, 1));
#pragma unroll
    for (int i = 0; i < KCH; ++i) kreg[i] = buf_load16(kr, koff[i]);
#pragma unroll
    for (int i = 0; i < VBL; ++i) {
      if (VTOT % NT != 0 && tid + NT * i >= VTOT) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[i][r] = buf_load16(vr, voff[i] + r * vrow);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) *(u32x4*)(&Ks[buf][kdst[i]]) = kreg[i];
#pragma unroll
    for (int i = 0; i < VBL; ++i) {
      if (VTOT % NT != 0 && tid + NT * i >= VTOT) continue;
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // columns 4 w .. 4 w + 3 of the 16
        const uint32_t rows[4] = {vreg[i][0][w], vreg[i][1][w], vreg[i][2][w], vreg[i][3][w]};
        uint32_t cols[4];
        transpose4x4_b8(rows, cols);
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) *(uint32_t*)(&Vt[buf][vdst[i] + (4 * w + c2) * VSTR]) = cols[c2];
      }
    }
  };

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
    if (__any(mx > m_run + kLazy8)) {
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
    // p * scale_p * 2^-kLazy8 = exp2(S * scale * log2e - m + log2(scale_p) -
    // kLazy8) in fp32: its sum is l * scale_p * 2^-kLazy8; its e4m3 rounding
    // is packed as the B operand, byte m = 16 nb + r of this lane half.
    const float off = lsp - kLazy8 - (m_run == -INFINITY ? 0.f : m_run);  // all -inf scores: P = 0
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
      const uint8_t* vr = &Vt[buf][(db * 32 + j) * VSTR + 32 * h];
      const u32x4 lo = *(const u32x4*)vr, hi = *(const u32x4*)(vr + 16);
      const i32x8 va = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      oacc[db] = mfma_fp8(va, pb, oacc[db]);
    }
  }

  const float l_tot = wave_sum_halves(l_run);  // = l * scale_p * 2^-kLazy8
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
      a.lse[((int64_t)bi * a.h_q + hq) * a.s_q + my_q] =
          live ? (m_run + __log2f(l_tot) - lsp + kLazy8) * kLn2 : -INFINITY;
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
