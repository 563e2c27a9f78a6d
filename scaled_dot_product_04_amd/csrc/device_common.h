// Device-side helpers shared by the gfx950 attention kernels: vector types,
// the 32x32x16 MFMA operand/accumulator conventions, and small LDS/global
// access helpers.
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_{bf16,f16}, wave64):
//   A operand (32 x 16): lane l holds row i = l % 32 and 8 consecutive
//     contraction indices selected by the lane half h = l / 32.
//   B operand (16 x 32): lane l holds column j = l % 32 and the same 8
//     contraction indices for its half h.
//   Accumulator (32 x 32 fp32, 16 registers): lane l holds column j = l % 32;
//     register r holds row 8 * (r / 4) + 4 * h + (r % 4).
// Only the pairing "A lane (i, h, m) meets B lane (j, h, m)" matters for a
// contraction, so any one-to-one assignment of (h, m) to contraction indices
// works as long as both operands use the same one. When an operand is built
// from an accumulator, its (h, m) -> index assignment is the accumulator's row
// layout, and the operand read from LDS follows it (see key_of()).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace sdpa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type traits for the 16-bit MFMA paths.
struct Bf16T {
  typedef __bf16 elem;
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
struct F16T {
  typedef _Float16 elem;
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even 16-bit and packed (low = x); one
// v_cvt_pk_{bf16,f16}_f32.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef typename T::elem E;
  typedef E E2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x, y}), E2));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N - 1 (unrolled at
// compile time, so array indices derived from i stay in registers).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// MFMA with its accumulator in AGPRs. The kernels are compiled with VGPR
// accumulators; this form keeps a long-lived accumulator out of the
// architectural VGPRs, and an MFMA whose accumulator is in AGPRs lets the
// vector work of the same wave issue beside it. The compiler does not track
// hazards into inline assembly: an operand written by a VALU instruction
// needs two wait states before the MFMA reads it. The callers feed LDS reads
// and values packed well before, and a test compiles the kernels to assembly
// and checks that no VALU write of an operand lands in the two instructions
// before one of these MFMAs. Readers of the accumulators must wait for the
// last MFMA (mfma_acc_drain).
template <typename T>
__device__ __forceinline__ void mfma_acc(f32x16& c, typename T::vec8 a, typename T::vec8 b);
template <>
__device__ __forceinline__ void mfma_acc<Bf16T>(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma_acc<F16T>(f32x16& c, f16x8 a, f16x8 b) {
  asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// 24 wait states: more than an MFMA result needs before a VALU or
// v_accvgpr_read reads it. The accumulators pass through empty statements
// ordered after the wait, so that no read of them moves above it (without
// them the compiler hoisted the epilogue's AGPR reads over the wait).
template <int N, typename... A>
__device__ __forceinline__ void mfma_acc_drain(f32x16 (&a0)[N], A&... rest) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  auto pin = [](f32x16 (&a)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+a"(a[i]));
  };
  pin(a0);
  (pin(rest), ...);
}

// Buffer resource for raw buffer loads of gfx9-class GPUs: `bytes` is the
// number of addressable bytes from `base`; loads at offsets >= bytes return 0.
// Base and size must be the same in every lane of the wave (they are read
// from the first lane, so the descriptor lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* up = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte pieces addressed by lanes 4 j + i / 4 of the group,
// j = 0..3 (one 16-bit value per j).
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Bytes of rows [row0, n_rows) of a row-major tile with `row_stride` elements
// between rows and `row_len` elements per row (0 if none), clamped to 2^31.
// Workgroup ids are dealt round-robin over the 8 XCDs (id % 8), each with its
// own L2. Maps a dispatch slot s in [0, total) to a work slot such that the
// `share` consecutive work slots that read the same K/V (the query heads of
// one KV group, or the splits of one) sit on one XCD and consecutive such
// groups go to different XCDs, so that unequal groups (a ragged batch) still
// spread over the whole chip. Identity when total or total / share is not a
// multiple of 8.
__device__ __forceinline__ int xcd_slot(int s, int total, int share) {
  if ((total & 7) != 0 || ((total / share) & 7) != 0) return s;
  const int x = s & 7, k = s >> 3;
  return (x + 8 * (k / share)) * share + k % share;
}

// Lengths of batch element bi under the padding mask: lq valid query rows,
// lk valid keys (per-batch device arrays, clamped to [0, s]; null = full), and
// the causal diagonal offset: key j is visible to row i iff j <= i + off, with
// off = lk - lq for bottom-right alignment, 0 for top-left. Uniform per block.
struct BatchLens {
  int lq, lk, off;
};
__device__ __forceinline__ BatchLens batch_lens(const int32_t* seq_q, const int32_t* seq_kv, int bi, int s_q,
                                                int s_kv, bool causal, int bottom_right) {
  BatchLens r;
  r.lq = seq_q ? min(max(__builtin_amdgcn_readfirstlane(seq_q[bi]), 0), s_q) : s_q;
  r.lk = seq_kv ? min(max(__builtin_amdgcn_readfirstlane(seq_kv[bi]), 0), s_kv) : s_kv;
  r.off = (causal && bottom_right) ? r.lk - r.lq : 0;
  return r;
}

__device__ __forceinline__ uint32_t tile_bytes(int row0, int n_rows, int64_t row_stride, int row_len,
                                               int elem_bytes) {
  if (row0 >= n_rows) return 0u;
  const int64_t b = ((int64_t)(n_rows - row0 - 1) * row_stride + row_len) * elem_bytes;
  return b > 0x7fffffffLL ? 0x7fffffffu : (uint32_t)b;
}

template <typename T>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  typedef typename T::elem E;
  return (float)__builtin_bit_cast(E, bits);
}

// Row of the 32x32 accumulator held by register r of a lane in half h.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

// Contraction index (within a 16-wide k-step t) that lane half h's element m
// stands for, when the operand is taken from accumulator registers
// 8*(t%2) .. 8*(t%2)+7 of accumulator block t/2:  16 t + 8 (m/4) + 4 h + m%4.
__device__ __forceinline__ constexpr int key_of(int t, int h, int m) {
  return 16 * t + 8 * (m / 4) + 4 * h + (m % 4);
}

// Max / sum of x over lanes l and l ^ 32 (the two halves holding the same
// accumulator column), in both lanes, through v_permlane32_swap (a VALU
// exchange: no LDS traffic, no LDS wait). The swap of a register pair (a, b),
// both holding x, leaves x of lanes 0..31 in both halves of a and x of lanes
// 32..63 in both halves of b. It is written in assembly because the compiler's
// builtin returns its first result for both outputs; the two wait states
// before it are the ones the compiler itself puts between a VALU write and the
// swap's read. Every lane of the wave must be active.
__device__ __forceinline__ f32x2 halves_swap(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
  return f32x2{lo, hi};
}
__device__ __forceinline__ float wave_max_halves(float x) {
  const f32x2 r = halves_swap(x);
  return fmaxf(r.x, r.y);
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  const f32x2 r = halves_swap(x);
  return r.x + r.y;
}

// Chunk swizzle of the row-major V tile: row r keeps its 16-byte chunk c at
// position c ^ vswz<D>(r). The LDS serves a 64-lane 8-byte read in two passes
// of 32 lanes over 64 banks (256 bytes); in one transposed read, the 32 lanes
// of a pass touch 4 consecutive rows x 2 column groups of 32 bytes each, and
// this XOR spreads them over all 16 chunk positions (D = 128: one row per 256
// bytes, rows 4k..4k+3 shifted by 0, 4, 8, 12 chunks; D = 64: two rows per 256
// bytes, row pairs shifted by 0 and 4). A pass of 16-byte row stores covers
// whole rows, which any XOR keeps conflict-free.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? (r & 3) << 2 : ((r >> 1) & 1) << 2;
}

// Lane offsets for transposed operand reads from a swizzled row-major tile of
// D columns (rows = keys): lane (column 32 db + l % 32, half h) receives rows
// 16 t + 4 h + 0..3 and 16 t + 8 + 4 h + 0..3 via two ds_read_b64_tr_b16.
template <int D>
struct SwzLaneF {
  int tr_off[D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int i = lane & 15, grp = lane >> 4, h = lane >> 5;
    const int row = 4 * h + (i >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * (grp & 1) + 4 * (i & 3);
      tr_off[db] = row * D + (((col >> 3) ^ vswz<D>(row)) * 8) + 4 * ((col >> 2) & 1);
    }
  }
  template <typename V8>
  __device__ __forceinline__ V8 tr(const uint16_t* tile, int db, int t) const {
    const uint16_t* p = &tile[tr_off[db] + 16 * t * D];
    const u32x2 lo = ds_read_tr16(p);
    const u32x2 hi = ds_read_tr16(p + 8 * D);
    return __builtin_bit_cast(V8, u32x4{lo.x, lo.y, hi.x, hi.y});
  }
};

// Score modifiers, in natural-log units (the caller multiplies by log2 e).
// bias_row points at bias[b][h][i][0] of one query row i (null: no bias).
// Four consecutive keys key..key+3 of that row; keys past n_keys read as 0
// (they are masked anyway; the guard only keeps the reads in bounds).
template <typename T>
__device__ __forceinline__ f32x4 bias4(const void* bias_row, int bias_f32, int key, int n_keys) {
  f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
  if (bias_row == nullptr) return r;
  if (key + 3 < n_keys) {
    if (bias_f32) return *(const f32x4*)((const float*)bias_row + key);
    const u32x2 w = *(const u32x2*)((const uint16_t*)bias_row + key);
    return f32x4{to_f32<T>((uint16_t)(w.x & 0xffff)), to_f32<T>((uint16_t)(w.x >> 16)),
                 to_f32<T>((uint16_t)(w.y & 0xffff)), to_f32<T>((uint16_t)(w.y >> 16))};
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (key + e < n_keys)
      r[e] = bias_f32 ? ((const float*)bias_row)[key + e] : to_f32<T>(((const uint16_t*)bias_row)[key + e]);
  return r;
}

// One bias value bias[row][key] (null row or out of range: 0).
template <typename T>
__device__ __forceinline__ float bias1(const void* bias_row, int bias_f32, int key, int n_keys) {
  if (bias_row == nullptr || key >= n_keys) return 0.f;
  return bias_f32 ? ((const float*)bias_row)[key] : to_f32<T>(((const uint16_t*)bias_row)[key]);
}

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): per round, (hi0, lo0) = M0 * c0 and
// (hi1, lo1) = M1 * c2 as 64-bit products, the counter becomes
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), and the key advances by (W0, W1).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // One 32 x 32 -> 64-bit product (v_mad_u64_u32) gives both halves.
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c2 = hi0 ^ c3 ^ k1;
    c1 = lo1;
    c3 = lo0;
  }
  return u32x4{c0, c1, c2, c3};
}

// The four words of the block (rows row4*4 .. +3, keys key4*4 .. +3).
__device__ __forceinline__ u32x4 drop_words(uint32_t key4, uint32_t row4, uint32_t slot, uint32_t offset,
                                            uint32_t seed_lo, uint32_t seed_hi) {
  return philox4x32_10(key4, row4, slot, offset, seed_lo, seed_hi);
}

__device__ __forceinline__ bool drop_keep(uint32_t word, int byte, int k8) {
  return (int)((word >> (8 * byte)) & 0xFFu) < k8;
}

// Four lanes that need the same four dropout blocks (a quad of consecutive
// query rows, or of consecutive keys) each draw one block and trade the
// parts the others need, instead of all four drawing all four.

// 4x4 transpose of dwords across the lanes of a quad (lanes 4m .. 4m+3): lane
// L holds a[0..3]; afterwards lane L holds out[k] = a[L] of lane k. Two
// rounds of DPP exchanges (lane ^ 1, then lane ^ 2) and selects.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ u32x4 quad_transpose(u32x4 a, int lane) {
  const bool b0 = lane & 1, b1 = lane & 2;
  const uint32_t x0 = dpp_xor1(a[1]), x1 = dpp_xor1(a[0]), x2 = dpp_xor1(a[3]), x3 = dpp_xor1(a[2]);
  u32x4 s;
  s[0] = b0 ? x0 : a[0];
  s[1] = b0 ? a[1] : x1;
  s[2] = b0 ? x2 : a[2];
  s[3] = b0 ? a[3] : x3;
  const uint32_t y0 = dpp_xor2(s[2]), y1 = dpp_xor2(s[3]), y2 = dpp_xor2(s[0]), y3 = dpp_xor2(s[1]);
  u32x4 r;
  r[0] = b1 ? y0 : s[0];
  r[1] = b1 ? y1 : s[1];
  r[2] = b1 ? s[2] : y2;
  r[3] = b1 ? s[3] : y3;
  return r;
}

// 4x4 transpose of the bytes of four dwords: out[t] byte w = in[w] byte t.
__device__ __forceinline__ u32x4 bytes_transpose4(u32x4 w) {
  const uint32_t p01l = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
  const uint32_t p01h = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
  const uint32_t p23l = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t p23h = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  return u32x4{__builtin_amdgcn_perm(p23l, p01l, 0x05040100u), __builtin_amdgcn_perm(p23l, p01l, 0x07060302u),
               __builtin_amdgcn_perm(p23h, p01h, 0x05040100u), __builtin_amdgcn_perm(p23h, p01h, 0x07060302u)};
}

}  // namespace sdpa
