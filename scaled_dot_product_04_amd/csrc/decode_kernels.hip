// Split-KV forward for few query rows against many keys (a KV-cache decode or
// prefill-chunk step), bf16 / fp16, d in {64, 128}.
//
// The JAX attention codelab (step 9, "MHA, GQA, MQA") motivates shared KV
// heads by the KV-cache memory of inference: in that regime the forward reads
// every K/V byte once per step, so the kernel is bound by HBM, not by the
// matrix cores. The work is laid out for that:
//  * All query heads of one KV group and all query positions form the rows of
//    one 32-row block (row = head_in_group * s_q + position), so K and V are
//    read once per KV head, not once per query head.
//  * The key range is split into chunks ("splits"); each one-wave workgroup
//    runs the online softmax of the forward over one chunk for one row block
//    and writes a partial (O / l, LSE) in fp32. A second kernel merges the
//    partials of each row: LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s
//    (the same row softmax, re-associated over the chunks).
//  * With one split the first kernel writes O and LSE directly.
// Masks and padding lengths follow the forward (per-batch lengths, top-left or
// bottom-right causal diagonal; rows that see no key: O = 0, LSE = -inf).
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

constexpr int kDecBN = 32;  // keys per K/V tile

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_decode_kernel(FwdArgs a, DecodeArgs dc) {
  typedef typename T::elem E;
  typedef typename T::vec8 V8;
  constexpr int BN = kDecBN;
  constexpr int KSTR = D + 8;         // LDS row stride (elements) of the K tile
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int KCH = BN * CH / 64;   // K (and V) chunks staged per lane
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];

  const int lane = threadIdx.x;
  const int j = lane & 31, h = lane >> 5;
  int id = blockIdx.x;  // splits of one row block are adjacent
  const int sp = id % dc.n_split;
  id /= dc.n_split;
  const int rb = id % dc.n_rb;
  id /= dc.n_rb;
  const int g = id % a.h_kv, bi = id / a.h_kv;
  const int G = a.h_q / a.h_kv;
  const BatchLens L = batch_lens(a.seq_q, a.seq_kv, bi, a.s_q, a.s_kv, CAUSAL, a.bottom_right);

  // This lane's row (its column of S^T): query head g*G + hl, position qi.
  const int row = rb * 32 + j;
  const int hl = row / a.s_q, qi = row - hl * a.s_q;
  const bool row_ok = hl < G;
  const int hq = g * G + (row_ok ? hl : 0);
  const bool live = row_ok && qi < L.lq;

  const E* qp = (const E*)a.q + bi * a.qs.b + hq * a.qs.h + (int64_t)qi * a.qs.s;
  V8 qf[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) qf[t] = live ? *(const V8*)(qp + 16 * t + 8 * h) : V8{};

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  // Keys of this split, clipped to the keys that some valid row can see (the
  // last valid row lq - 1 sees keys <= lq - 1 + off). Keys past k_end belong
  // to the next split and are masked even when a tile reads them.
  const int kv_hi = CAUSAL ? max(0, min(L.lk, L.lq + L.off)) : L.lk;
  const int k_begin = sp * dc.split_keys;
  const int k_end = min(k_begin + dc.split_keys, kv_hi);
  const int n_tiles = k_end > k_begin ? (k_end - k_begin + BN - 1) / BN : 0;

  const E* kp = (const E*)a.k + bi * a.ks.b + g * a.ks.h;
  const E* vp = (const E*)a.v + bi * a.vs.b + g * a.vs.h;
  uint32_t koff[KCH], kdst[KCH], voff[KCH], vdst[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = lane + 64 * i;
    const int r = c / CH, cc = c % CH;
    koff[i] = (uint32_t)(r * a.ks.s * 2 + cc * 16);
    kdst[i] = r * KSTR + cc * 8;
    voff[i] = (uint32_t)(r * a.vs.s * 2 + cc * 16);
    vdst[i] = r * D + ((cc ^ vswz<D>(r)) * 8);
  }
  SwzLaneF<D> sl;
  sl.init(lane);
  u32x4 kreg[KCH], vreg[KCH];
  auto load_tile = [&](int k0) {  // rows at or past lk read as zero
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + (int64_t)k0 * a.ks.s, tile_bytes(k0, L.lk, a.ks.s, D, 2));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + (int64_t)k0 * a.vs.s, tile_bytes(k0, L.lk, a.vs.s, D, 2));
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

  if (n_tiles > 0) {
    load_tile(k_begin);
    store_tile(0);
    if (n_tiles > 1) load_tile(k_begin + BN);
  }
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int k0 = k_begin + tile * BN;
    const int buf = tile & 1;
    __syncthreads();  // the wave's LDS writes of this buffer are complete
    if (tile + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (tile + 2 < n_tiles) load_tile(k0 + 2 * BN);
    }
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int t = 0; t < NKS; ++t) {
      const V8 kf = *(const V8*)(&Ks[buf][j * KSTR + 16 * t + 8 * h]);
      sacc = T::mfma(kf, qf[t], sacc);
    }
    if ((k0 + BN > k_end) || (CAUSAL && k0 + BN - 1 > L.off)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + acc_row(r, h);
        if (key >= k_end || (CAUSAL && key > qi + L.off)) sacc[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = wave_max_halves(mx) * sl2;
    if (__any(mx > m_run + 8.f)) {  // lazy rescale, as in the forward
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    const float msub = m_run == -INFINITY ? 0.f : m_run;
    uint32_t pk[8];
    float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[r], sl2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], sl2, -msub));
      lsum0 += p0;
      lsum1 += p1;
      pk[r / 2] = pack2<T>(p0, p1);
    }
    l_run += lsum0 + lsum1;
#pragma unroll
    for (int t2 = 0; t2 < BN / 16; ++t2) {
      const V8 pb = __builtin_bit_cast(V8, u32x4{pk[4 * t2], pk[4 * t2 + 1], pk[4 * t2 + 2], pk[4 * t2 + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = T::mfma(sl.template tr<V8>(Vs[buf], db, t2), pb, oacc[db]);
    }
  }

  const float l_tot = wave_sum_halves(l_run);
  const bool has = live && l_tot > 0.f;
  const float inv = has ? 1.f / l_tot : 0.f;
  const float lse = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!row_ok) return;
  if (dc.n_split == 1) {
    E* op = (E*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)qi * a.os.s;
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
    if (a.lse != nullptr && h == 0) a.lse[((int64_t)bi * a.h_q + hq) * a.s_q + qi] = lse;
  } else {
    const int64_t prow = (((int64_t)sp * a.b + bi) * a.h_q + hq) * a.s_q + qi;
    float* po = dc.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = db * 32 + 8 * rq + 4 * h;
        *(f32x4*)(po + d0) = f32x4{oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv,
                                   oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv};
      }
    if (h == 0) dc.part_lse[prow] = lse;
  }
}

// Merges the split partials of each row: one thread per (row, 4 columns), in
// 64-thread blocks (few rows: spread over many compute units); the loads of
// the split loops are unrolled so that several are in flight.
template <typename T, int D>
__global__ __launch_bounds__(64) void fwd_decode_combine_kernel(FwdArgs a, DecodeArgs dc) {
  typedef typename T::elem E;
  constexpr int PER = D / 4;
  const int64_t rows = (int64_t)a.b * a.h_q * a.s_q;
  const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int64_t row = t / PER;
  const int c4 = (int)(t % PER) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < dc.n_split; ++s) mx = fmaxf(mx, dc.part_lse[s * rows + row]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {  // some split saw a key
    float sum = 0.f;
#pragma unroll 8
    for (int s = 0; s < dc.n_split; ++s) {
      const float w = __builtin_amdgcn_exp2f((dc.part_lse[s * rows + row] - mx) * kLog2e);
      sum += w;
      acc += w * *(const f32x4*)(dc.part_o + (s * rows + row) * D + c4);
    }
    acc *= 1.f / sum;
    lse = mx + __logf(sum);
  }
  const int qi = (int)(row % a.s_q);
  const int64_t bh = row / a.s_q;
  const int hq = (int)(bh % a.h_q), bi = (int)(bh / a.h_q);
  E* op = (E*)a.o + bi * a.os.b + hq * a.os.h + (int64_t)qi * a.os.s + c4;
  *(u32x2*)op = u32x2{pack2<T>(acc[0], acc[1]), pack2<T>(acc[2], acc[3])};
  if (a.lse != nullptr && c4 == 0) a.lse[row] = lse;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, const DecodeArgs& dc, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.b * a.h_kv * dc.n_rb * dc.n_split)), block(64);
  if (a.causal)
    hipLaunchKernelGGL((fwd_decode_kernel<T, D, true>), grid, block, 0, stream, a, dc);
  else
    hipLaunchKernelGGL((fwd_decode_kernel<T, D, false>), grid, block, 0, stream, a, dc);
  if (dc.n_split > 1) {
    const int64_t threads = (int64_t)a.b * a.h_q * a.s_q * (D / 4);
    hipLaunchKernelGGL((fwd_decode_combine_kernel<T, D>), dim3((unsigned)((threads + 63) / 64)), dim3(64), 0,
                       stream, a, dc);
  }
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int b, int h_q, int h_kv, int s_q, int s_kv, int d, Io io) {
  DecodePlan p{};
  if (!(io == Io::BF16 || io == Io::F16) || !(d == 64 || d == 128) || b <= 0 || s_q <= 0) return p;
  const int G = h_q / h_kv;
  const int64_t rows = (int64_t)G * s_q;
  const int n_rb = (int)((rows + 31) / 32);
  // The row-block forward reads a KV head's K/V once per query head, with
  // s_q of its 128 or 256 rows in use; this path reads them once per 32-row
  // block. It is taken for long key ranges when that is no more traffic
  // (row blocks <= query heads per KV head) and the query rows are few.
  if (s_q > 64 || s_kv < 512 || n_rb > G) return p;
  // About 2048 one-wave workgroups (4 resident per CU by LDS: two rounds),
  // and at least 256 keys per split.
  const int64_t blocks = (int64_t)b * h_kv * n_rb;
  int64_t n_split = (2048 + blocks - 1) / blocks;
  n_split = n_split < (s_kv + 255) / 256 ? n_split : (s_kv + 255) / 256;
  if (n_split < 1) n_split = 1;
  const int split_keys = (int)(((s_kv + n_split - 1) / n_split + kDecBN - 1) / kDecBN * kDecBN);
  p.use = true;
  p.n_rb = n_rb;
  p.split_keys = split_keys;
  p.n_split = (s_kv + split_keys - 1) / split_keys;
  const size_t prow = (size_t)b * h_q * s_q;
  p.ws_bytes = p.n_split > 1 ? align256((size_t)p.n_split * prow * d * sizeof(float)) +
                                   (size_t)p.n_split * prow * sizeof(float)
                             : 0;
  return p;
}

hipError_t launch_fwd_decode(const FwdArgs& a, const DecodePlan& p, void* workspace, Io io, hipStream_t stream) {
  DecodeArgs dc{};
  dc.n_split = p.n_split;
  dc.split_keys = p.split_keys;
  dc.n_rb = p.n_rb;
  if (p.n_split > 1) {
    const size_t prow = (size_t)a.b * a.h_q * a.s_q;
    dc.part_o = (float*)workspace;
    dc.part_lse = (float*)((char*)workspace + align256((size_t)p.n_split * prow * a.d * sizeof(float)));
  }
  if (io == Io::BF16) return a.d == 64 ? launch_d<Bf16T, 64>(a, dc, stream) : launch_d<Bf16T, 128>(a, dc, stream);
  return a.d == 64 ? launch_d<F16T, 64>(a, dc, stream) : launch_d<F16T, 128>(a, dc, stream);
}

}  // namespace sdpa
