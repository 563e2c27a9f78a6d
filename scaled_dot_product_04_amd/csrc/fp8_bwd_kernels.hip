// FP8 backward: the exact-gradient backward of the fused attention with every
// matrix product on the fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Recipe: the HYBRID format of the JAX attention codelab (step 10): q, k, v in
// e4m3 as in the forward, the incoming gradient dO in e5m2, each with a
// per-tensor factor (real value = code * descale); the recipe's delayed
// scaling derives those factors from a history of per-tensor absolute maxima.
// The gradient formulas are those of the 16-bit backward:
//   P = exp(scale * Q K^T - LSE),  D_i = sum_d dO_id O_id,
//   dP = dO V^T,  dS = P * (dP - D),
//   dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
// The five products run on fp8 operands with fp32 accumulation:
//   S = Q K^T      e4m3 x e4m3 codes (exact products)
//   dP = dO V^T    dO's format x e4m3
//   dV = P^T dO    P quantised to e4m3 as P * scale_p (P <= 1, so the largest
//                  weight maps to scale_p <= 448) x dO's format
//   dK = dS^T Q    dS quantised as dS * scale_ds, saturated to the format's
//   dQ = dS K      largest finite value, x e4m3
// with every per-tensor factor folded into the fp32 scalars applied to the
// accumulators. dS is quantised to e4m3 by default or to e5m2 (the format the
// recipe names for backward-pass tensors); scale_ds is the caller's (from its
// amax history), and the dK/dV kernel reports max |dS| for that history.
//
// Layout trick shared by both kernels. An operand built from accumulator
// registers holds, in lane half h, the 16 accumulator rows 8 (r/4) + 4 h + r%4
// of each 32-row block. The A operand of the score products is loaded with
// lane i holding tile row pi(i) = 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3)
// (the tiles are stored in LDS with row pi(i) at position i), so accumulator
// register r of lane half h is tile row 16 h + r: the 32 contraction values of
// half h are the two 16-row runs 16 h .. 16 h + 15 and 32 + 16 h .. + 15 of a
// 64-row tile, and the matching transposed operand is two plain 16-byte reads.
//
// Kernels, in launch order (atomic-free except the one max per wave for the
// amax report; deterministic):
//  1. dQ: query-stationary (8 waves x 32 query rows); K / V tiles of 64 keys
//     stream through LDS (K row-major and transposed, V row-major). It also
//     writes D = rowsum(dO * O) for the second kernel.
//  2. dK/dV: key-stationary (8 waves x 32 keys; the wave's K and V rows stay in
//     registers); 64-row Q / dO tiles stream through LDS row-major and are
//     also read transposed (ds_read_b64_tr_b8). Query-head groups that would underfill the GPU are split
//     and reduced as in the 16-bit backward.
#include <type_traits>

#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kT8 = 64;        // rows per streamed tile (one 64-deep contraction)
constexpr int kNT8 = 512;      // threads per workgroup (8 waves)
constexpr int kKeys8 = 128;    // keys per dK/dV workgroup (4 x 32, each with a dV and a dK wave)
constexpr int kRows8 = 256;    // query rows per dQ workgroup

// Format codes of the f8f6f4 MFMA operands: 0 = e4m3, 1 = e5m2.
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
}

// Largest finite value of the dS format.
template <bool E5M2>
__device__ __forceinline__ constexpr float fp8_max() { return E5M2 ? 57344.f : 448.f; }

// Four fp32 values (already scaled) rounded to the fp8 format and packed, byte e = x[e].
template <bool E5M2>
__device__ __forceinline__ uint32_t pack4_fp8(float x0, float x1, float x2, float x3) {
  // The low-half convert keeps the upper 16 bits of its old value, which the
  // high-half convert overwrites: any register serves (x0's bits).
  const int old = (int)__float_as_uint(x0);
  if constexpr (E5M2) {
    const int w = __builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, old, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(x2, x3, w, true);
  } else {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, old, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  }
}

// Position (LDS row) of tile row q in a row-major tile read as an A operand:
// the inverse of pi within each 32-row block.
__device__ __forceinline__ constexpr int pi_pos(int q) {
  return 32 * (q >> 5) + 8 * ((q >> 2) & 3) + 4 * ((q >> 4) & 1) + (q & 3);
}

// LDS geometry of one 64-row fp8 tile of D columns, row-major (the A operand
// of the score products, and through transposed reads of the dV, dK and dQ
// products): pitch D + 16 bytes, row q at position pi_pos(q); 16 lanes
// reading one 16-byte column chunk of 16 consecutive positions hit 16
// distinct 4-bank groups (36 dwords apart).
template <int D>
struct Geo8 {
  static constexpr int RSTR = D + 16;
  static constexpr int ROW_BYTES = kT8 * RSTR;
  static constexpr int BPT = (kT8 / 4) * (D / 8);  // 4-row x 8-byte blocks per tile
};

// One 4-row x 8-byte block (rows 4 rg .. 4 rg + 3, bytes 8 cg .. 8 cg + 7) of
// a 64-row fp8 tile in flight, loaded with buffer loads (rows past the end
// read as zero) and stored row-major.
template <int D>
struct Blk8 {
  typedef Geo8<D> G;
  u32x2 r[4];
  uint32_t goff;  // byte offset of the block's first row, relative to the tile's first row
  int rdst;       // row-major LDS offset of its first row (pi_pos(4 rg + e) = pi_pos(4 rg) + e)
  __device__ __forceinline__ void init(int t, int64_t stride) {
    const int rg = t / (D / 8), cg = t % (D / 8);
    goff = (uint32_t)(4 * rg * stride + 8 * cg);
    rdst = pi_pos(4 * rg) * G::RSTR + 8 * cg;
  }
  __device__ __forceinline__ void load(const uint8_t* tile0, int row0, int n_rows, int64_t stride) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile0, tile_bytes(row0, n_rows, stride, D, 1));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, goff + (uint32_t)(e * stride), 0, 0));
  }
  __device__ __forceinline__ void store_rows(uint8_t* tile) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) *(u32x2*)(&tile[rdst + e * G::RSTR]) = r[e];
  }
};

__device__ __forceinline__ i32x8 lds_op32(const uint8_t* p) {
  const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// ds_read_b64_tr_b8: within each 16-lane group, lane i receives byte i % 8
// of the 8-byte pieces addressed by lanes 2 k + i / 8 of the group, k = 0..7
// (byte k of the result from piece k).
__device__ __forceinline__ u32x2 ds_read_tr8(const uint8_t* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p)));
}

// Transposed A operand (column block of a row-major tile, contraction over the
// tile's 64 rows) read straight from the row-major tile: lane (column j, half
// h) gets the rows 16 h .. 16 h + 15 and 32 + 16 h .. 32 + 16 h + 15 in order,
// which sit at positions pi_pos() = 16 u + 8 (k / 4) + 4 h + k % 4 for byte
// 8 u + k. Lane l of 16-lane group G addresses position 8 (k / 4) +
// 4 (G / 2) + k % 4 (k = (l % 16) / 2) at columns 16 (G % 2) + 8 (l % 2) of
// the block (tr_lane_off); the four reads are 16 positions apart.
template <int D>
__device__ __forceinline__ int tr_lane_off(int lane) {
  const int G = lane >> 4, L = lane & 15, k = L >> 1;
  return (8 * (k >> 2) + 4 * (G >> 1) + (k & 3)) * Geo8<D>::RSTR + 16 * (G & 1) + 8 * (L & 1);
}
template <int D>
__device__ __forceinline__ i32x8 lds_tr_op(const uint8_t* p) {
  constexpr int P16 = 16 * Geo8<D>::RSTR;
  const u32x2 r0 = ds_read_tr8(p), r1 = ds_read_tr8(p + P16), r2 = ds_read_tr8(p + 2 * P16), r3 = ds_read_tr8(p + 3 * P16);
  return i32x8{(int)r0.x, (int)r0.y, (int)r1.x, (int)r1.y, (int)r2.x, (int)r2.y, (int)r3.x, (int)r3.y};
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// A workgroup owns 128 keys. Waves 0..3 (role dV) and 4..7 (role dK) share
// them: wave w and wave w + 4 both own keys 32 (w % 4) .. + 31 and run on the
// same SIMD. Per 64-row tile t:
//   dV wave: S = Q K^T, P (masked), dV^T += dO^T P; it also leaves P * scale_p
//            (fp16, lane-private layout) in LDS for its dK partner;
//   dK wave: one tile behind: dS for tile t - 1 from that P and the dP it
//            formed at the previous step, dK^T += Q^T dS; then dP = dO V^T
//            for tile t, held in registers until P(t) arrives.
// So every product is formed once (16 MFMAs per tile and key slice), each
// wave holds one accumulator set (64 registers), the exponentials are taken
// once, and one barrier per tile still orders everything: P(t) is written
// before the barrier that starts step t + 1, where the dK wave reads it. The
// Q tile and D values stay one step longer (three buffers). The transposed
// operands (Q^T of dK, dO^T of dV) are read from the row-major tiles with
// ds_read_b64_tr_b8. Masked scores give P = 0, hence dS = 0: the dK wave
// needs no mask.
template <int D, bool CAUSAL, bool DO_E5M2, bool DS_E5M2, bool AMAX>
__global__ __launch_bounds__(kNT8, 1) void bwd8_dkdv_kernel(BwdArgs a, int n_split, float* part) {
  typedef Geo8<D> G;
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  constexpr int NKS = D / 64, NDB = D / 32;
  constexpr int FDO = DO_E5M2 ? 1 : 0, FDS = DS_E5M2 ? 1 : 0;
  static_assert(2 * G::BPT <= kNT8 && G::BPT <= kNT8 / 2, "staging map");
  // P exchange: per key slice, 64 lanes x 32 fp16 (64 bytes) at an 80-byte
  // pitch (16 lanes storing one 16-byte piece each hit distinct 4-bank groups).
  constexpr int PXP = 80, PXS = 64 * PXP;
  // Row-major Q (three deep: the dK wave reads a tile's Q^T one step after
  // its S) and dO tiles; the transposed operands are read from them.
  __shared__ __attribute__((aligned(16))) uint8_t Qr[3][G::ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Dr[2][G::ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Px[2][4 * PXS];
  __shared__ __attribute__((aligned(16))) float lse2s[2][kT8];
  __shared__ __attribute__((aligned(16))) float dels[3][kT8];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const bool role_dk = wu >= 4;
  const int kw = wu & 3;  // key slice of this wave
  const int n_slots = a.b * a.h_kv * n_split;
  const int kb = blockIdx.x / n_slots;
  const int slot = xcd_slot(blockIdx.x - kb * n_slots, n_slots, n_split);
  const int sp = slot % n_split;
  const int bg = slot / n_split;
  const int g = bg % a.h_kv, bi = bg / a.h_kv;
  const int G_ = a.h_q / a.h_kv, Gs = G_ / n_split;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const int kw0 = kb * kKeys8 + kw * 32;
  const int my_key = kw0 + j;
  // This lane's K row (dV wave: B operand of S) or V row (dK wave: of dP),
  // bytes 64 t + 32 h .. + 31; keys at or past lk read as zero.
  i32x8 kvf[NKS];
  {
    const int k0 = kb * kKeys8;
    const Strides3 st = role_dk ? a.vs : a.ks;
    const uint8_t* base = (const uint8_t*)(role_dk ? a.v : a.k) + bi * st.b + g * st.h + (int64_t)k0 * st.s;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, tile_bytes(k0, L.lk, st.s, D, 1));
#pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const uint32_t o = (uint32_t)((kw * 32 + j) * st.s + 64 * t + 32 * h);
      const u32x4 x0 = buf_load16(rs, o), x1 = buf_load16(rs, o + 16);
      kvf[t] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
  }
  f32x16 acc[NDB];  // dV^T (role dV) or dK^T (role dK)
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  f32x16 dph[2];  // dK wave: dP of the tile whose P is still to come
  dph[0] = dph[1] = f32x16{};
  // Weights are produced pre-multiplied by scale_p (the log2 of it is folded
  // into the exponent), and dS * scale_ds as p' * (dP' - D') with the
  // factors folded: dP' = dp_acc * dp_scale * scale_ds / scale_p, D' = D *
  // scale_ds / scale_p.
  const float sl2 = a.scale * kLog2e;
  const float lsp = __log2f(a.f8.scale_p);
  const float dpf = a.f8.dp_scale * a.f8.scale_ds / a.f8.scale_p;
  const float dlf = a.f8.scale_ds / a.f8.scale_p;
  constexpr float FMAX = fp8_max<DS_E5M2>();
  float amax = 0.f;  // max |dS * scale_ds| of this lane (role dK)
  // An addend of 0 the compiler cannot see as a constant: with it, p' * t
  // with p' in fp16 is one v_fma_mix_f32 (a plain product would convert p'
  // first).
  float zero;
  asm("s_mov_b32 %0, 0" : "=s"(zero));

  const int n_qt = (L.lq + kT8 - 1) / kT8;
  const int qt0 = CAUSAL ? min(n_qt, max(0, kb * kKeys8 - L.off) / kT8) : 0;
  const int nq = kb * kKeys8 >= L.lk ? 0 : n_qt - qt0;
  const int n_it = Gs * nq;
  const int hq_base = g * G_ + sp * Gs;

  // Staging: waves [0, BPT / 64) carry blocks of the Q tile, waves [4, 4 +
  // BPT / 64) blocks of the dO tile; threads [0, 64) also the tile's LSE and
  // D values. The choice is made per wave (readfirstlane), so that the tile's
  // buffer descriptor stays uniform: a per-lane choice between the two
  // descriptors would turn each load into a waterfall loop that waits for it.
  const bool st_q = wu < G::BPT / 64, st_d = wu >= 4 && wu - 4 < G::BPT / 64;
  const uint8_t* const stage_base = st_q ? (const uint8_t*)a.q + bi * a.qs.b : (const uint8_t*)a.dout + bi * a.dos.b;
  const Strides3 stage_st = st_q ? a.qs : a.dos;
  Blk8<D> blk;
  blk.init(st_q ? tid : tid - kNT8 / 2, stage_st.s);
  float lreg = 0.f, creg = 0.f;
  bool lvalid = false;
  // Tiles are walked query head by query head (hq_base ..), each over query
  // tiles qt0 .. qt0 + nq - 1. Running cursors (no division per tile): the
  // next tile to load and the tile being computed.
  int ld_hq = hq_base, ld_qt = qt0;
  auto load_tile = [&]() {
    const int hq = ld_hq;
    const int q0 = ld_qt * kT8;
    if (++ld_qt == qt0 + nq) {
      ld_qt = qt0;
      ++ld_hq;
    }
    if (st_q || st_d) blk.load(stage_base + hq * stage_st.h + (int64_t)q0 * stage_st.s, q0, L.lq, stage_st.s);
    if (tid < kT8) {  // rows past lq read row lq - 1 (any valid row) and are zeroed when staged
      const int qi = q0 + tid;
      lvalid = qi < L.lq;
      const int64_t row = ((int64_t)bi * a.h_q + hq) * a.s_q + min(qi, L.lq - 1);
      lreg = a.lse[row];
      creg = a.delta[row];
    }
  };
  auto store_tile = [&](int b2, int b3) {
    if (st_q)
      blk.store_rows(Qr[b3]);
    else if (st_d)
      blk.store_rows(Dr[b2]);
    if (tid < kT8) {
      // A row that sees no key has LSE = -inf and every score masked; 0 keeps
      // exp2(-inf - lse) at 0 instead of NaN.
      lse2s[b2][tid] = (lvalid && lreg != -INFINITY) ? lreg * kLog2e - lsp : 0.f;
      dels[b3][tid] = lvalid ? creg * dlf : 0.f;
    }
  };

  // Per-lane LDS offsets: A-operand row j of each 32-row block, the
  // transposed reads (tr_lane_off; column block db 32 db bytes further), and
  // this lane's P exchange slot.
  const int rowoff = j * G::RSTR + 32 * h;
  const int troff = tr_lane_off<D>(lane);
  const int pxoff = kw * PXS + lane * PXP;

  // dK wave: dS and dK for the tile whose dP is in dph, P in Px[pb], Q in
  // Qr[b3], D in dels[b3].
  auto dk_finish = [&](int pb, int b3) __attribute__((always_inline)) {
    // Read as eight fp16 values per 16 bytes. (Bit-casting single 32-bit
    // elements of a 4 x u32 vector to two fp16 values and converting them has
    // been compiled into reads of element 0 only.)
    f16x8 pw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pw[c] = __builtin_bit_cast(f16x8, *(const u32x4*)(&Px[pb][pxoff + 16 * c]));
    uint32_t sk[8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int row0 = 32 * nb + 16 * h + 4 * w;
        const f32x4 d4 = *(const f32x4*)(&dels[b3][row0]);
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)  // dS * scale_ds
          ds[e] = fmaf((float)pw[2 * nb + w / 2][4 * (w % 2) + e], fmaf(dph[nb][4 * w + e], dpf, -d4[e]), zero);
        // The reported maximum is taken before saturation, so that a scale
        // history sees the values that did not fit.
        if (AMAX) amax = fmaxf(amax, fmaxf(fmaxf(fabsf(ds[0]), fabsf(ds[1])), fmaxf(fabsf(ds[2]), fabsf(ds[3]))));
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[e] = __builtin_amdgcn_fmed3f(ds[e], -FMAX, FMAX);
        sk[4 * nb + w] = pack4_fp8<DS_E5M2>(ds[0], ds[1], ds[2], ds[3]);
      }
    const i32x8 sb = i32x8{(int)sk[0], (int)sk[1], (int)sk[2], (int)sk[3], (int)sk[4], (int)sk[5], (int)sk[6], (int)sk[7]};
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = mfma8<0, FDS>(lds_tr_op<D>(&Qr[b3][troff + 32 * db]), sb, acc[db]);
  };

  if (n_it > 0) {
    load_tile();
    store_tile(0, 0);
    if (n_it > 1) load_tile();
  }
  int cur_qt = qt0 - 1;
  int b3 = 0;             // buffer of the tile being computed among the three-deep ones
  bool prev_live = false;  // the previous tile had work for this key slice (dK wave)
  // Start of iteration `it`, the same in both roles (every wave meets the
  // same barriers): advance the tile cursor, barrier, stage the next tile.
  auto begin_tile = [&](int it, int& q0) {
    const int buf = it & 1;
    const int b3n = b3 == 2 ? 0 : b3 + 1;
    cur_qt = cur_qt + 1 == qt0 + nq ? qt0 : cur_qt + 1;
    q0 = cur_qt * kT8;
    __syncthreads();  // tile `it` and P of tile it - 1 are in LDS; nothing still reads the buffers written next
    if (it + 1 < n_it) {
      store_tile(buf ^ 1, b3n);
      if (it + 2 < n_it) load_tile();
    }
  };
  // Each role runs its own loop, so that its accumulators are updated in one
  // place: with both roles' updates in one loop body the compiler gave them
  // two register ranges and copied the 64 accumulator registers from one to
  // the other and back every tile.
  if (role_dk) {
    for (int it = 0; it < n_it; ++it) {
      const int buf = it & 1;
      const int b3n = b3 == 2 ? 0 : b3 + 1, b3p = b3 == 0 ? 2 : b3 - 1;
      int q0;
      begin_tile(it, q0);
      // A tile whose queries all precede this slice's keys has no work.
      const bool live = !(CAUSAL && q0 + kT8 - 1 + L.off < kw0);
      if (prev_live) dk_finish(buf ^ 1, b3p);
      if (live) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f32x16 dp = f32x16{};
#pragma unroll
          for (int t = 0; t < NKS; ++t)
            dp = mfma8<FDO, 0>(lds_op32(&Dr[buf][nb * 32 * G::RSTR + rowoff + 64 * t]), kvf[t], dp);
          dph[nb] = dp;
        }
      }
      prev_live = live;
      b3 = b3n;
    }
  } else {
    for (int it = 0; it < n_it; ++it) {
      const int buf = it & 1;
      const int b3n = b3 == 2 ? 0 : b3 + 1;
      int q0;
      begin_tile(it, q0);
      const bool live = !(CAUSAL && q0 + kT8 - 1 + L.off < kw0);
      if (live) {
        const bool need_mask = (q0 + kT8 > L.lq) || (kw0 + 32 > L.lk) || (CAUSAL && q0 + L.off < kw0 + 31);
        // The body exists with and without the mask, each one branch-free: a
        // mask branch inside it would split it into blocks across which the
        // hoisted operand reads stay live.
        auto dv_body = [&](auto masked) __attribute__((always_inline)) -> i32x8 {
          constexpr bool MASKED = decltype(masked)::value;
          uint32_t pk[8];
          u32x4 ph[4];  // P * scale_p as fp16 pairs, for the dK wave
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            // S for tile rows 32 nb + 16 h + r (register r) x this lane's key.
            f32x16 s = f32x16{};
#pragma unroll
            for (int t = 0; t < NKS; ++t)
              s = mfma8<0, 0>(lds_op32(&Qr[b3][nb * 32 * G::RSTR + rowoff + 64 * t]), kvf[t], s);
            if (MASKED) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int qi = q0 + 32 * nb + 16 * h + r;
                if (qi >= L.lq || my_key >= L.lk || (CAUSAL && my_key > qi + L.off)) s[r] = -INFINITY;
              }
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const f32x4 l4 = *(const f32x4*)(&lse2s[buf][32 * nb + 16 * h + 4 * w]);
              float p[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s[4 * w + e], sl2, -l4[e]));  // P * scale_p
              pk[4 * nb + w] = pack4_fp8<false>(p[0], p[1], p[2], p[3]);
              ph[2 * nb + w / 2][2 * (w % 2)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p[0], p[1]));
              ph[2 * nb + w / 2][2 * (w % 2) + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p[2], p[3]));
            }
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) *(u32x4*)(&Px[buf][pxoff + 16 * c]) = ph[c];
          return i32x8{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
        };
        const i32x8 pb = need_mask ? dv_body(std::true_type{}) : dv_body(std::false_type{});
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = mfma8<FDO, 0>(lds_tr_op<D>(&Dr[buf][troff + 32 * db]), pb, acc[db]);
      }
      b3 = b3n;
    }
  }
  // The last tile's dS: its P was written in the last step.
  __syncthreads();
  if (role_dk && prev_live) dk_finish((n_it - 1) & 1, b3 == 0 ? 2 : b3 - 1);

  if (AMAX && role_dk) {
    // One max per wave; non-negative floats order as their bit patterns.
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if (lane == 0) atomicMax((unsigned int*)a.f8.amax_ds, __float_as_uint(amax / a.f8.scale_ds));
  }
  if (my_key >= a.s_kv) return;
  const float osc = role_dk ? a.dk_scale : a.dv_scale;
  if (n_split == 1) {
    uint16_t* op = role_dk ? (uint16_t*)a.dk + bi * a.dks.b + g * a.dks.h + (int64_t)my_key * a.dks.s
                           : (uint16_t*)a.dv + bi * a.dvs.b + g * a.dvs.h + (int64_t)my_key * a.dvs.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 wv;
        wv.x = pack2<Bf16T>(acc[db][4 * rq] * osc, acc[db][4 * rq + 1] * osc);
        wv.y = pack2<Bf16T>(acc[db][4 * rq + 2] * osc, acc[db][4 * rq + 3] * osc);
        *(u32x2*)(op + d0) = wv;
      }
  } else {
    // fp32 partials: part[2][n_split][b][h_kv][s_kv][D] (dK first, then dV)
    const int64_t plane = (int64_t)a.b * a.h_kv * a.s_kv * D;
    const int64_t off = (int64_t)sp * plane + (((int64_t)bi * a.h_kv + g) * a.s_kv + my_key) * D;
    float* pp = part + (role_dk ? 0 : (int64_t)n_split * plane) + off;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        *(f32x4*)(pp + d0) = f32x4{acc[db][4 * rq] * osc, acc[db][4 * rq + 1] * osc, acc[db][4 * rq + 2] * osc,
                                   acc[db][4 * rq + 3] * osc};
      }
  }
}

// ---------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool DO_E5M2, bool DS_E5M2>
__global__ __launch_bounds__(kNT8, 1) void bwd8_dq_kernel(BwdArgs a, int n_qblk) {
  typedef Geo8<D> G;
  constexpr int NKS = D / 64, NDB = D / 32;
  constexpr int FDO = DO_E5M2 ? 1 : 0, FDS = DS_E5M2 ? 1 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t Kr[2][G::ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Vr[2][G::ROW_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int j = lane & 31, h = lane >> 5;
  const int bh_total = a.b * a.h_q;
  const int rank = blockIdx.x / bh_total;
  const int slot = xcd_slot(blockIdx.x - rank * bh_total, bh_total, a.h_q / a.h_kv);  // KV group: one XCD
  const int qb = n_qblk - 1 - rank;
  const int bi = slot / a.h_q, hq = slot - (slot / a.h_q) * a.h_q;
  const int g = hq / (a.h_q / a.h_kv);
  const int qblk0 = qb * kRows8;
  const int q0 = qblk0 + wave * 32;
  const int my_q = q0 + j;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  const uint8_t* qp = (const uint8_t*)a.q + bi * a.qs.b + hq * a.qs.h;
  const uint8_t* dop = (const uint8_t*)a.dout + bi * a.dos.b + hq * a.dos.h;
  const uint8_t* kp = (const uint8_t*)a.k + bi * a.ks.b + g * a.ks.h;
  const uint8_t* vp = (const uint8_t*)a.v + bi * a.vs.b + g * a.vs.h;

  // This lane's Q and dO row bytes 64 t + 32 h .. + 31 (B operands).
  i32x8 qf[NKS], df[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    if (my_q < L.lq) {
      const uint8_t* qr = qp + (int64_t)my_q * a.qs.s + 64 * t + 32 * h;
      const uint8_t* dr = dop + (int64_t)my_q * a.dos.s + 64 * t + 32 * h;
      const u32x4 q0v = *(const u32x4*)qr, q1v = *(const u32x4*)(qr + 16);
      const u32x4 d0v = *(const u32x4*)dr, d1v = *(const u32x4*)(dr + 16);
      qf[t] = i32x8{(int)q0v.x, (int)q0v.y, (int)q0v.z, (int)q0v.w, (int)q1v.x, (int)q1v.y, (int)q1v.z, (int)q1v.w};
      df[t] = i32x8{(int)d0v.x, (int)d0v.y, (int)d0v.z, (int)d0v.w, (int)d1v.x, (int)d1v.y, (int)d1v.z, (int)d1v.w};
    } else {
      qf[t] = i32x8{};
      df[t] = i32x8{};
    }
  }
  const int64_t row_bh = ((int64_t)bi * a.h_q + hq) * a.s_q;
  // Rows past lq have Q = dO = 0, so their dS and dQ are 0. A row that sees
  // no key has LSE = -inf and every score masked: 0 keeps its P at 0.
  const float lse = my_q < L.lq ? a.lse[row_bh + my_q] : 0.f;
  const float lsp = __log2f(a.f8.scale_p);
  const float lse2 = (lse == -INFINITY ? 0.f : lse * kLog2e) - lsp;
  // D = rowsum(dO * O) of this row: this lane holds dO bytes 64 t + 32 h ..
  // + 31 and reads the same columns of O; the halves are summed across the
  // wave. D = delta_scale * sum(code * O); the dK/dV kernel reads it from the
  // workspace (rows past lq hold 0 and are never used).
  float dpart = 0.f;
  if (my_q < L.lq) {
    const uint16_t* op = (const uint16_t*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)my_q * a.os.s;
#pragma unroll
    for (int t = 0; t < NKS; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // 8 codes (two words of df) against 8 bf16 values of O
        const u32x4 ov = *(const u32x4*)(op + 64 * t + 32 * h + 8 * c);
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
          const int word = df[t][2 * c + wd];
          const f32x2 f0 = DO_E5M2 ? __builtin_amdgcn_cvt_pk_f32_bf8(word, false)
                                   : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
          const f32x2 f1 = DO_E5M2 ? __builtin_amdgcn_cvt_pk_f32_bf8(word, true)
                                   : __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
          const uint32_t o0 = ov[2 * wd], o1 = ov[2 * wd + 1];
          dpart = fmaf(f0.x, __uint_as_float(o0 << 16), dpart);
          dpart = fmaf(f0.y, __uint_as_float(o0 & 0xffff0000u), dpart);
          dpart = fmaf(f1.x, __uint_as_float(o1 << 16), dpart);
          dpart = fmaf(f1.y, __uint_as_float(o1 & 0xffff0000u), dpart);
        }
      }
  }
  const float dl = wave_sum_halves(dpart) * a.delta_scale;
  if (h == 0 && my_q < a.s_q) a.delta[row_bh + my_q] = dl;
  const float sl2 = a.scale * kLog2e;
  const float dpf = a.f8.dp_scale * a.f8.scale_ds / a.f8.scale_p;
  const float dlf = dl * a.f8.scale_ds / a.f8.scale_p;
  constexpr float FMAX = fp8_max<DS_E5M2>();

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

  const int rowoff = j * G::RSTR + 32 * h;
  const int troff = tr_lane_off<D>(lane);  // K^T reads from the row-major K tile

  const int kv_end = qblk0 >= L.lq ? 0 : CAUSAL ? max(0, min(L.lk, min(qblk0 + kRows8, L.lq) + L.off)) : L.lk;
  const int n_tiles = (kv_end + kT8 - 1) / kT8;
  // Staging: waves [0, BPT / 64) carry blocks of the K tile, waves [4, 4 +
  // BPT / 64) blocks of the V tile (both row-major);
  // chosen per wave so that the buffer descriptor stays uniform.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const bool st_k = wu < G::BPT / 64, st_v = wu >= 4 && wu - 4 < G::BPT / 64;
  const uint8_t* const stage_base = st_k ? kp : vp;
  const int64_t stage_s = st_k ? a.ks.s : a.vs.s;
  Blk8<D> blk;
  blk.init(st_k ? tid : tid - kNT8 / 2, stage_s);
  auto load_tile = [&](int k0) {
    if (st_k || st_v) blk.load(stage_base + (int64_t)k0 * stage_s, k0, L.lk, stage_s);
  };
  auto store_tile = [&](int buf) {
    if (st_k)
      blk.store_rows(Kr[buf]);
    else if (st_v)
      blk.store_rows(Vr[buf]);
  };
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    if (n_tiles > 1) load_tile(kT8);
  }
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    const int k0 = tile * kT8;
    __syncthreads();  // buffer `buf` is complete; buffer buf ^ 1 is no longer read
    if (tile + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (tile + 2 < n_tiles) load_tile((tile + 2) * kT8);
    }
    if (CAUSAL && k0 > q0 + 31 + L.off) continue;  // every key of the tile is above this wave's rows
    const bool need_mask = (k0 + kT8 > L.lk) || (CAUSAL && k0 + kT8 - 1 > q0 + L.off);
    uint32_t sk[8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // S^T and dP^T for keys k0 + 32 nb + 16 h + r (register r) x this lane's query.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        s = mfma8<0, 0>(lds_op32(&Kr[buf][nb * 32 * G::RSTR + rowoff + 64 * t]), qf[t], s);
        dp = mfma8<0, FDO>(lds_op32(&Vr[buf][nb * 32 * G::RSTR + rowoff + 64 * t]), df[t], dp);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * nb + 16 * h + r;
          if (key >= L.lk || (CAUSAL && key > my_q + L.off)) s[r] = -INFINITY;
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[4 * w + e], sl2, -lse2));  // P * scale_p
          ds[e] = __builtin_amdgcn_fmed3f(p * fmaf(dp[4 * w + e], dpf, -dlf), -FMAX, FMAX);  // dS * scale_ds
        }
        sk[4 * nb + w] = pack4_fp8<DS_E5M2>(ds[0], ds[1], ds[2], ds[3]);
      }
    }
    const i32x8 sb = i32x8{(int)sk[0], (int)sk[1], (int)sk[2], (int)sk[3], (int)sk[4], (int)sk[5], (int)sk[6], (int)sk[7]};
    // dQ^T += K^T dS^T over the tile's 64 keys.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      dq[db] = mfma8<0, FDS>(lds_tr_op<D>(&Kr[buf][troff + 32 * db]), sb, dq[db]);
  }
  if (my_q < a.s_q) {
    uint16_t* dqp = (uint16_t*)a.dq + bi * a.dqs.b + hq * a.dqs.h + (int64_t)my_q * a.dqs.s;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        u32x2 w;
        w.x = pack2<Bf16T>(dq[db][4 * rq] * a.dq_scale, dq[db][4 * rq + 1] * a.dq_scale);
        w.y = pack2<Bf16T>(dq[db][4 * rq + 2] * a.dq_scale, dq[db][4 * rq + 3] * a.dq_scale);
        *(u32x2*)(dqp + d0) = w;
      }
  }
}

template <int D, bool CAUSAL, bool DO_E5M2, bool DS_E5M2>
hipError_t launch_fmt(const BwdArgs& a, hipStream_t stream, const TimingEvents& te) {
  const bool timed = te.n >= 3;
  if (timed) (void)hipEventRecord(te.ev[0], stream);
  const int n_qblk = (a.s_q + kRows8 - 1) / kRows8;
  hipLaunchKernelGGL((bwd8_dq_kernel<D, CAUSAL, DO_E5M2, DS_E5M2>), dim3(n_qblk * a.b * a.h_q), dim3(kNT8), 0,
                     stream, a, n_qblk);
  if (timed) (void)hipEventRecord(te.ev[1], stream);
  const int n_split = bwd_split_count(a.b, a.h_q, a.h_kv, a.s_kv, kKeys8);
  float* part = n_split > 1 ? bwd_partials(a) : nullptr;
  const int n_kblk = (a.s_kv + kKeys8 - 1) / kKeys8;
  const dim3 grid(n_kblk * a.b * a.h_kv * n_split);
  if (a.f8.amax_ds != nullptr)
    hipLaunchKernelGGL((bwd8_dkdv_kernel<D, CAUSAL, DO_E5M2, DS_E5M2, true>), grid, dim3(kNT8), 0, stream, a, n_split,
                       part);
  else
    hipLaunchKernelGGL((bwd8_dkdv_kernel<D, CAUSAL, DO_E5M2, DS_E5M2, false>), grid, dim3(kNT8), 0, stream, a, n_split,
                       part);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && n_split > 1) e = launch_bwd_reduce(a, n_split, part, stream);
  if (timed) (void)hipEventRecord(te.ev[2], stream);
  return e;
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream, const TimingEvents& te) {
  const bool c = a.causal != 0, de = a.f8.do_e5m2 != 0, se = a.f8.ds_e5m2 != 0;
  if (c) {
    if (de) return se ? launch_fmt<D, true, true, true>(a, stream, te) : launch_fmt<D, true, true, false>(a, stream, te);
    return se ? launch_fmt<D, true, false, true>(a, stream, te) : launch_fmt<D, true, false, false>(a, stream, te);
  }
  if (de) return se ? launch_fmt<D, false, true, true>(a, stream, te) : launch_fmt<D, false, true, false>(a, stream, te);
  return se ? launch_fmt<D, false, false, true>(a, stream, te) : launch_fmt<D, false, false, false>(a, stream, te);
}

}  // namespace

hipError_t launch_bwd_fp8(const BwdArgs& a, hipStream_t stream, const TimingEvents& te) {
  return a.d == 64 ? launch_d<64>(a, stream, te) : launch_d<128>(a, stream, te);
}

}  // namespace sdpa
