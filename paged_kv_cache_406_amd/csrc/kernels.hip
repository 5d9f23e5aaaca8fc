// Device side of the paged KV-cache library for gfx950 (CDNA4).
//
// Kernels
//   append_kernel      new tokens' K/V into their slots (bit copy, or FP8
//                      quantise-on-write with per-channel inverse scales)
//   copy_blocks_kernel whole-block copies for copy-on-write
//   decode_kernel      decode attention over the paged cache: per-wavefront
//                      ranges of (KV head, sequence, block) work, QK^T and PV
//                      on MFMA, online softmax in registers
//   merge_kernel       log-sum-exp merge of the partial results of sequences
//                      whose blocks were split across wavefronts
//
// Pages followed: "AI 陪读顶会论文（三）：KV Cache 显存占用计算与 PagedAttention
// 原理拆解" (section "为什么自回归解码…必须使用 KV Cache": the attention
// equation and the append of the new token's k, v; section
// "PagedAttention 的破局哲学": blocks, tables, copy-on-write) and
// "生成一个字，为什么要背一整本账" (section "显存账本": grouped-query heads;
// section "再往后：压 KV 的三条路线": FP8 with per-channel scales, the sliding
// window; the whole cache is read from HBM for every generated token).
//
// Design notes (gfx950)
//  * Decode is bound by HBM reads: every KV byte is used once per call.  One
//    wavefront owns a (KV head, sequence, block range); each 16-token
//    sub-tile of K and V goes from HBM straight into MFMA operand registers
//    and is used for all G query heads of the group at once (the GQA reuse).
//  * QK^T: S[16 tokens][16 heads] += K[16 tokens][k] * Q^T[k][16 heads] with
//    v_mfma_f32_16x16x16 (bf16 / f16) or 16x16x4 (f32).  Query heads beyond G
//    are zero columns.  The S layout (lane = head column, 4 token rows per
//    lane) is exactly the B operand PV needs, so P never moves between lanes.
//  * PV: O^T[16 dims][16 heads] += V^T[16 dims][16 tokens] * P^T[16 tokens][16 heads].
//    V is stored channel-major inside a block so that a lane's 4 tokens of one
//    channel are contiguous.  bf16 P is split into hi + lo bf16 parts (two
//    MFMAs) so the rounding of P stays far below fp32 accumulation error.
//  * The max of each head's scores is shared by the 4 lanes holding that head
//    (two lane exchanges); sums stay per lane until the end.
//  * Work split: all blocks of all (KV head, sequence) pairs are laid end to
//    end (KV-head major) and cut into W equal ranges, one per wavefront.  A
//    range that covers a whole sequence writes the final output; the pieces of
//    a sequence that straddles ranges are written as (unnormalised o, max,
//    sum) and combined by merge_kernel.  Workgroups are remapped so that each
//    XCD (one L2) gets a contiguous run of ranges.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "pool_internal.h"

namespace pkv {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum { KV_F32 = PKV_F32, KV_F16 = PKV_F16, KV_BF16 = PKV_BF16, KV_FP8 = PKV_FP8_E4M3 };

template <int KV> struct Elem;
template <> struct Elem<KV_F32> { static constexpr int bytes = 4; };
template <> struct Elem<KV_F16> { static constexpr int bytes = 2; };
template <> struct Elem<KV_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<KV_FP8> { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h;
  uint16_t s = (uint16_t)b;
  __builtin_memcpy(&h, &s, 2);
  return (float)h;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  uint16_t s;
  __builtin_memcpy(&s, &h, 2);
  return s;
}

// fp32 -> OCP E4M3, round to nearest even, saturating to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448 (and inf) saturate
  if (a >= 0x3c800000u) {                    // >= 2^-6: normal E4M3
    // keep 3 of the 23 mantissa bits, ties to even; the carry moves into the
    // exponent; rebias 127 -> 7.  Inputs < 448 cannot round past 448.
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
  }
  // subnormal range: value = m * 2^-9, m in 0..8 (8 is the smallest normal)
  const float scaled = __uint_as_float(a) * 512.0f;  // exact
  return sign | (uint32_t)__builtin_rintf(scaled);
}

template <int SRC>
__device__ __forceinline__ float src_to_f32(const uint8_t* p, int64_t idx);
template <> __device__ __forceinline__ float src_to_f32<KV_F32>(const uint8_t* p, int64_t idx) {
  return reinterpret_cast<const float*>(p)[idx];
}
template <> __device__ __forceinline__ float src_to_f32<KV_F16>(const uint8_t* p, int64_t idx) {
  return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[idx]);
}
template <> __device__ __forceinline__ float src_to_f32<KV_BF16>(const uint8_t* p, int64_t idx) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[idx]);
}

// four E4M3 codes (one dword) -> four bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ s16x4 e4m3x4_to_bf16x4(uint32_t codes) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
  s16x4 r;
  __builtin_memcpy(&r, &lo, 4);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 4, &hi, 4);
  return r;
}

// ---------------------------------------------------------------------------
// append: tokens [n][Hkv][D] -> pool slots
// ---------------------------------------------------------------------------
struct AppendParams {
  uint8_t* kc;
  uint8_t* vc;
  const uint8_t* k;
  const uint8_t* v;
  const int64_t* slots;
  const float* k_inv;
  const float* v_inv;
  int64_t num_blocks;
  int32_t n, hkv, d, bs, layer;
};

template <int KV, int SRC>
__global__ __launch_bounds__(256) void append_kernel(AppendParams P) {
  constexpr int EB = Elem<KV>::bytes;
  constexpr int X = 16 / EB;
  const int chunks = P.d / X;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)P.n * P.hkv * chunks;
  if (t >= total) return;
  const int c = (int)(t % chunks);
  const int h = (int)((t / chunks) % P.hkv);
  const int64_t i = t / ((int64_t)chunks * P.hkv);
  const int64_t slot = P.slots[i];
  if (slot < 0 || slot >= P.num_blocks * P.bs) return;
  const int64_t blk = slot / P.bs;
  const int off = (int)(slot % P.bs);
  const int64_t tile = ((int64_t)P.layer * P.num_blocks + blk) * P.hkv + h;
  const int64_t src0 = (i * P.hkv + h) * P.d + (int64_t)c * X;  // element index
  uint8_t* kdst = P.kc + ((tile * (P.d / X) + c) * P.bs + off) * 16;
  uint8_t* vdst = P.vc + (tile * P.d + (int64_t)c * X) * P.bs * EB + (int64_t)off * EB;
  if constexpr (KV == SRC) {
    const uint4 kv = *reinterpret_cast<const uint4*>(P.k + src0 * EB);
    *reinterpret_cast<uint4*>(kdst) = kv;
    const uint8_t* vs = P.v + src0 * EB;
#pragma unroll
    for (int e = 0; e < X; ++e) {
      uint8_t* dst = vdst + (int64_t)e * P.bs * EB;
      if constexpr (EB == 4) *reinterpret_cast<uint32_t*>(dst) = reinterpret_cast<const uint32_t*>(vs)[e];
      else if constexpr (EB == 2) *reinterpret_cast<uint16_t*>(dst) = reinterpret_cast<const uint16_t*>(vs)[e];
    }
  } else {
    static_assert(KV == KV_FP8, "only same-dtype copy or FP8 quantisation");
    const int64_t s0 = ((int64_t)P.layer * P.hkv + h) * P.d + (int64_t)c * X;
    uint32_t kw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < X; ++e) {
      const float kx = src_to_f32<SRC>(P.k, src0 + e) * P.k_inv[s0 + e];
      const float vx = src_to_f32<SRC>(P.v, src0 + e) * P.v_inv[s0 + e];
      kw[e >> 2] |= f32_to_e4m3(kx) << (8 * (e & 3));
      vdst[(int64_t)e * P.bs] = (uint8_t)f32_to_e4m3(vx);
    }
    *reinterpret_cast<uint4*>(kdst) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
  }
}

// ---------------------------------------------------------------------------
// copy-on-write: whole blocks, every layer, K and V
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* kc, uint8_t* vc,
                                                          const kv_block_copy* pairs,
                                                          int64_t num_blocks, int64_t tile_bytes) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  uint8_t* base = blockIdx.z == 0 ? kc : vc;
  const int32_t src = pairs[pair].src;
  const int32_t dst = pairs[pair].dst;
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
  const uint4* s = reinterpret_cast<const uint4*>(base + ((int64_t)layer * num_blocks + src) * tile_bytes);
  uint4* d = reinterpret_cast<uint4*>(base + ((int64_t)layer * num_blocks + dst) * tile_bytes);
  const int64_t n16 = tile_bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
struct DecodeParams {
  const uint8_t* kc;
  const uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* q;
  uint8_t* out;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_o;    // [W][2][G][D]
  float* ws_ml;   // [W][2][G][2]
  int64_t num_blocks;
  int32_t layer, batch, hq, hkv, group, max_blocks, window, out_dtype;
  int32_t num_waves;   // W (range mode)
  int32_t single;      // 1: one wavefront per (sequence, KV head)
  int32_t xcd_remap;
  float scale_log2;    // scale * log2(e)
};

// Blocks of sequence b that the query attends (window applied).
template <int BS>
__device__ __forceinline__ void seq_extent(const DecodeParams& P, int b, int32_t* L_out,
                                           int32_t* lo_out, int32_t* first_out, int32_t* nblk_out) {
  int32_t L = P.lens[b];
  const int32_t cap = P.max_blocks * BS;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int32_t lo = P.window > 0 ? (L - P.window > 0 ? L - P.window : 0) : 0;
  const int32_t first = lo / BS;
  *L_out = L;
  *lo_out = lo;
  *first_out = first;
  *nblk_out = L > lo ? (L + BS - 1) / BS - first : 0;
}

// Exclusive prefix sums of the per-sequence block counts into C[0..B] (LDS).
template <int BS>
__device__ void scan_block_counts(const DecodeParams& P, int32_t* C) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  const int per = (P.batch + 255) / 256;
  const int b0 = tid * per;
  const int b1 = min(P.batch, b0 + per);
  int32_t local = 0;
  for (int b = b0; b < b1; ++b) {
    int32_t L, lo, first, nb;
    seq_extent<BS>(P, b, &L, &lo, &first, &nb);
    local += nb;
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - local;
  for (int b = b0; b < b1; ++b) {
    int32_t L, lo, first, nb;
    seq_extent<BS>(P, b, &L, &lo, &first, &nb);
    C[b] = run;
    run += nb;
  }
  if (tid == 255) C[P.batch] = part[255];
  __syncthreads();
}

__device__ __forceinline__ int64_t range_start(int64_t w, int64_t T, int64_t W) { return w * T / W; }

// Largest w with range_start(w) <= x (the wavefront whose range holds x).
__device__ __forceinline__ int64_t wave_of(int64_t x, int64_t T, int64_t W) {
  return ((x + 1) * W - 1) / T;
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Operand / load types per KV dtype.
template <int KV> struct Ops;
template <> struct Ops<KV_F32> {
  typedef float qop;          // one k-step of 16x16x4 f32
  typedef uint4 vload;        // 4 tokens of one channel
  static constexpr int kpl = 1;
};
template <> struct Ops<KV_F16> {
  typedef f16x4 qop;
  typedef uint2 vload;
  static constexpr int kpl = 4;
};
template <> struct Ops<KV_BF16> {
  typedef s16x4 qop;
  typedef uint2 vload;
  static constexpr int kpl = 4;
};
template <> struct Ops<KV_FP8> {
  typedef s16x4 qop;
  typedef uint32_t vload;
  static constexpr int kpl = 4;
};

template <int KV, int D, int BS>
struct Decoder {
  static constexpr int EB = Elem<KV>::bytes;
  static constexpr int X = 16 / EB;          // channels per 16-byte K group
  static constexpr int NCH = D / (4 * X);    // 16-byte K loads per lane per sub-tile
  static constexpr int NV = D / 16;          // V loads (channel groups) per lane per sub-tile
  static constexpr int STEPS = D / (4 * Ops<KV>::kpl);  // QK MFMA steps
  static constexpr int SUB = BS / 16;        // 16-token sub-tiles per block
  typedef typename Ops<KV>::qop qop;
  typedef typename Ops<KV>::vload vload;

  // channel held by element e (0 .. D/4-1) of lane group kg's K vector
  static __device__ __forceinline__ int chan(int kg, int e) { return (kg + 4 * (e / X)) * X + (e % X); }

  // Loads this lane's q operands (head i of group g; zero for i >= G).  FP8
  // folds the per-channel K scale into q (q'[c] = q[c] * k_scale[c]).
  static __device__ __forceinline__ void load_q(const DecodeParams& P, int b, int g, int i, int kg,
                                                qop (&qo)[STEPS]) {
    const bool live = i < P.group;
    const int64_t row = ((int64_t)b * P.hq + (int64_t)g * P.group + (live ? i : 0)) * D;
    if constexpr (KV == KV_F32) {
      const float* q = reinterpret_cast<const float*>(P.q) + row;
#pragma unroll
      for (int s = 0; s < STEPS; ++s) qo[s] = live ? q[chan(kg, s)] : 0.0f;
    } else if constexpr (KV == KV_F16 || KV == KV_BF16) {
      const uint16_t* q = reinterpret_cast<const uint16_t*>(P.q) + row;
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        s16x4 v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = live ? (short)q[chan(kg, 4 * s + u)] : (short)0;
        __builtin_memcpy(&qo[s], &v, 8);
      }
    } else {
      const uint16_t* q = reinterpret_cast<const uint16_t*>(P.q) + row;
      const float* ks = P.k_scale + ((int64_t)P.layer * P.hkv + g) * D;
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        s16x4 v;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = chan(kg, 4 * s + u);
          const float x = live ? bf16_bits_to_f32(q[c]) * ks[c] : 0.0f;
          v[u] = (short)f32_to_bf16_bits_rne(x);
        }
        qo[s] = v;
      }
    }
  }

  struct Tile {
    uint4 k[NCH];
    vload v[NV];
  };

  static __device__ __forceinline__ void load_tile(Tile& t, const uint8_t* kblk, const uint8_t* vblk,
                                                   int st, int i, int kg) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      t.k[j] = *reinterpret_cast<const uint4*>(kblk + ((int64_t)((kg + 4 * j) * BS + 16 * st + i) * X) * EB);
#pragma unroll
    for (int n = 0; n < NV; ++n)
      t.v[n] = *reinterpret_cast<const vload*>(vblk + ((int64_t)(16 * n + i) * BS + 16 * st + 4 * kg) * EB);
  }

  static __device__ __forceinline__ f32x4 qk(const Tile& t, const qop (&qo)[STEPS]) {
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const float kf[4] = {__uint_as_float(t.k[j].x), __uint_as_float(t.k[j].y),
                             __uint_as_float(t.k[j].z), __uint_as_float(t.k[j].w)};
#pragma unroll
        for (int u = 0; u < 4; ++u) S = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[u], qo[4 * j + u], S, 0, 0, 0);
      }
    } else if constexpr (KV == KV_F16 || KV == KV_BF16) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const uint2 lo = make_uint2(t.k[j].x, t.k[j].y);
        const uint2 hi = make_uint2(t.k[j].z, t.k[j].w);
        qop a0, a1;
        __builtin_memcpy(&a0, &lo, 8);
        __builtin_memcpy(&a1, &hi, 8);
        if constexpr (KV == KV_F16) {
          S = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, qo[2 * j], S, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, qo[2 * j + 1], S, 0, 0, 0);
        } else {
          S = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, qo[2 * j], S, 0, 0, 0);
          S = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, qo[2 * j + 1], S, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const uint32_t w4[4] = {t.k[j].x, t.k[j].y, t.k[j].z, t.k[j].w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          S = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(e4m3x4_to_bf16x4(w4[u]), qo[4 * j + u], S, 0, 0, 0);
      }
    }
    return S;
  }

  // Zero the V elements of tokens r with !valid[r] (their bits may be garbage).
  static __device__ __forceinline__ void mask_v(Tile& t, const bool (&valid)[4]) {
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if constexpr (KV == KV_F32) {
        if (!valid[0]) t.v[n].x = 0;
        if (!valid[1]) t.v[n].y = 0;
        if (!valid[2]) t.v[n].z = 0;
        if (!valid[3]) t.v[n].w = 0;
      } else if constexpr (KV == KV_F16 || KV == KV_BF16) {
        const uint32_t m0 = (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
        const uint32_t m1 = (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
        t.v[n].x &= m0;
        t.v[n].y &= m1;
      } else {
        const uint32_t m = (valid[0] ? 0xffu : 0u) | (valid[1] ? 0xff00u : 0u) |
                           (valid[2] ? 0xff0000u : 0u) | (valid[3] ? 0xff000000u : 0u);
        t.v[n] &= m;
      }
    }
  }

  static __device__ __forceinline__ void pv(const Tile& t, const float (&p)[4], f32x4 (&O)[NV]) {
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const float vf[4] = {__uint_as_float(t.v[n].x), __uint_as_float(t.v[n].y),
                             __uint_as_float(t.v[n].z), __uint_as_float(t.v[n].w)};
#pragma unroll
        for (int u = 0; u < 4; ++u) O[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[u], p[u], O[n], 0, 0, 0);
      }
    } else if constexpr (KV == KV_F16) {
      f16x4 ph;
#pragma unroll
      for (int u = 0; u < 4; ++u) ph[u] = (_Float16)p[u];
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        f16x4 a;
        __builtin_memcpy(&a, &t.v[n], 8);
        O[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, ph, O[n], 0, 0, 0);
      }
    } else {
      // p = hi + lo, both bf16 (hi = round(p), lo = round(p - hi))
      const f32x2 p01 = {p[0], p[1]};
      const f32x2 p23 = {p[2], p[3]};
      const bf16x2 h01 = __builtin_convertvector(p01, bf16x2);
      const bf16x2 h23 = __builtin_convertvector(p23, bf16x2);
      const f32x2 r01 = p01 - __builtin_convertvector(h01, f32x2);
      const f32x2 r23 = p23 - __builtin_convertvector(h23, f32x2);
      const bf16x2 l01 = __builtin_convertvector(r01, bf16x2);
      const bf16x2 l23 = __builtin_convertvector(r23, bf16x2);
      s16x4 phi, plo;
      __builtin_memcpy(&phi, &h01, 4);
      __builtin_memcpy(reinterpret_cast<char*>(&phi) + 4, &h23, 4);
      __builtin_memcpy(&plo, &l01, 4);
      __builtin_memcpy(reinterpret_cast<char*>(&plo) + 4, &l23, 4);
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        s16x4 a;
        if constexpr (KV == KV_BF16) {
          __builtin_memcpy(&a, &t.v[n], 8);
        } else {
          a = e4m3x4_to_bf16x4(t.v[n]);
        }
        O[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, O[n], 0, 0, 0);
        O[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, O[n], 0, 0, 0);
      }
    }
  }

  // One (KV head g, sequence b) piece: logical blocks [first + j0, first + j1).
  // full: the piece is the whole attended range -> write the final output;
  // otherwise write the partial to workspace slot (w, which).
  static __device__ void piece(const DecodeParams& P, int b, int g, int j0, int j1, bool full,
                               int64_t w, int which) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int kg = lane >> 4;
    int32_t L, lo, first, nb;
    seq_extent<BS>(P, b, &L, &lo, &first, &nb);
    L = uniform(L);
    lo = uniform(lo);
    first = uniform(first);

    qop qo[STEPS];
    load_q(P, b, g, i, kg, qo);

    f32x4 O[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float lsum = 0.f;

    const int32_t* trow = P.tables + (int64_t)b * P.max_blocks;
    const int64_t tile_elems = (int64_t)D * BS;
    for (int j = j0; j < j1; ++j) {
      const int blk = first + j;
      const int32_t pb = uniform(trow[blk]);
      if (pb < 0 || pb >= P.num_blocks) continue;
      const int64_t tile = ((int64_t)P.layer * P.num_blocks + pb) * P.hkv + g;
      const uint8_t* kblk = P.kc + tile * tile_elems * EB;
      const uint8_t* vblk = P.vc + tile * tile_elems * EB;
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
        const int32_t t0 = blk * BS + 16 * st;
        if (t0 + 16 <= lo || t0 >= L) continue;
        Tile t;
        load_tile(t, kblk, vblk, st, i, kg);
        const f32x4 S = qk(t, qo);
        // Masking is branch-free: a branch between the QK MFMAs and the first
        // read of S would leave the MFMA-to-VALU wait states to the branch
        // target.
        float s[4];
        bool valid[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t tok = t0 + 4 * kg + r;
          valid[r] = tok >= lo && tok < L;
          s[r] = valid[r] ? S[r] * P.scale_log2 : -INFINITY;
        }
        mask_v(t, valid);
        float bmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        const float m_new = fmaxf(m, bmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
        lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m = m_new;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int n = 0; n < NV; ++n) O[n] *= alpha;
        }
        pv(t, p, O);
      }
    }
    const float ltot = lsum + __shfl_xor(lsum, 16);
    const float lall = ltot + __shfl_xor(ltot, 32);

    // channel scale of V (FP8) and the output position
    float vsc[NV][4];
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) vsc[n][r] = 1.0f;
    if constexpr (KV == KV_FP8) {
      const float* vs = P.v_scale + ((int64_t)P.layer * P.hkv + g) * D;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const f32x4 sc = *reinterpret_cast<const f32x4*>(vs + 16 * n + 4 * kg);
#pragma unroll
        for (int r = 0; r < 4; ++r) vsc[n][r] = sc[r];
      }
    }
    if (i >= P.group) return;
    if (full) {
      const float inv = lall > 0.f ? 1.0f / lall : 0.f;
      const int64_t row = ((int64_t)b * P.hq + (int64_t)g * P.group + i) * D;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = O[n][r] * inv * vsc[n][r];
        const int64_t off = row + 16 * n + 4 * kg;
        if (P.out_dtype == PKV_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.out) + off) = f32x4{o[0], o[1], o[2], o[3]};
        } else if (P.out_dtype == PKV_BF16) {
          const uint2 pk = make_uint2(f32_to_bf16_bits_rne(o[0]) | (f32_to_bf16_bits_rne(o[1]) << 16),
                                      f32_to_bf16_bits_rne(o[2]) | (f32_to_bf16_bits_rne(o[3]) << 16));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + off) = pk;
        } else {
          const uint2 pk = make_uint2(f32_to_f16_bits(o[0]) | (f32_to_f16_bits(o[1]) << 16),
                                      f32_to_f16_bits(o[2]) | (f32_to_f16_bits(o[3]) << 16));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + off) = pk;
        }
      }
    } else {
      const int64_t slot = (w * 2 + which) * P.group + i;
      float* wo = P.ws_o + slot * D;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = O[n][r] * vsc[n][r];
        *reinterpret_cast<f32x4*>(wo + 16 * n + 4 * kg) = o;
      }
      if (kg == 0) *reinterpret_cast<f32x2*>(P.ws_ml + slot * 2) = f32x2{m, lall};
    }
  }
};

template <int D>
__device__ __forceinline__ void write_zero_rows(const DecodeParams& P, int b, int g, int lane) {
  // G rows of D outputs for (b, g)
  const int64_t row0 = ((int64_t)b * P.hq + (int64_t)g * P.group) * D;
  const int64_t n = (int64_t)P.group * D;
  for (int64_t e = lane; e < n; e += 64) {
    if (P.out_dtype == PKV_F32) reinterpret_cast<float*>(P.out)[row0 + e] = 0.f;
    else reinterpret_cast<uint16_t*>(P.out)[row0 + e] = 0;
  }
}

template <int KV, int D, int BS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams P) {
  typedef Decoder<KV, D, BS> Dec;
  extern __shared__ int32_t C[];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int64_t wg = blockIdx.x;
  if (P.xcd_remap) wg = (wg % 8) * (gridDim.x / 8) + wg / 8;
  const int64_t w = wg * 4 + wid;

  if (P.single) {
    // one wavefront per (KV head, sequence), KV-head major
    if (w >= (int64_t)P.hkv * P.batch) return;
    const int g = (int)(w / P.batch);
    const int b = (int)(w % P.batch);
    int32_t L, lo, first, nb;
    seq_extent<BS>(P, b, &L, &lo, &first, &nb);
    if (nb == 0) {
      write_zero_rows<D>(P, b, g, lane);
      return;
    }
    Dec::piece(P, b, g, 0, nb, true, 0, 0);
    return;
  }

  scan_block_counts<BS>(P, C);
  const int64_t t_head = C[P.batch];
  const int64_t T = t_head * P.hkv;
  const int64_t W = P.num_waves;
  if (w >= W || T == 0) return;
  const int64_t r0 = range_start(w, T, W);
  const int64_t r1 = range_start(w + 1, T, W);
  int64_t x = r0;
  while (x < r1) {
    const int g = (int)(x / t_head);
    const int32_t r = (int32_t)(x % t_head);
    // largest b with C[b] <= r; blocks of b are [C[b], C[b+1])
    int lo_b = 0, hi_b = P.batch - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (C[mid] <= r) lo_b = mid;
      else hi_b = mid - 1;
    }
    const int b = uniform(lo_b);
    const int32_t cb = uniform(C[b]);
    const int32_t nb = uniform(C[b + 1]) - cb;
    const int32_t j0 = r - cb;
    const int64_t seg_end = x - j0 + nb;
    const int64_t pend = seg_end < r1 ? seg_end : r1;
    const int32_t j1 = j0 + (int32_t)(pend - x);
    const bool full = j0 == 0 && j1 == nb;
    Dec::piece(P, b, g, j0, j1, full, w, x == r0 ? 0 : 1);
    x = pend;
  }
}

// One wavefront per (KV head, sequence): zero an empty sequence, or combine
// the pieces of a sequence whose blocks straddle wavefront ranges.
template <int D, int BS>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams P) {
  extern __shared__ int32_t C[];
  scan_block_counts<BS>(P, C);
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= (int64_t)P.hkv * P.batch) return;
  const int g = (int)(seg / P.batch);
  const int b = (int)(seg % P.batch);
  const int32_t nb = C[b + 1] - C[b];
  if (nb == 0) {
    write_zero_rows<D>(P, b, g, lane);
    return;
  }
  const int64_t t_head = C[P.batch];
  const int64_t T = t_head * P.hkv;
  const int64_t W = P.num_waves;
  const int64_t s0 = (int64_t)g * t_head + C[b];
  const int64_t s1 = s0 + nb;
  const int64_t wf = wave_of(s0, T, W);
  const int64_t wl = wave_of(s1 - 1, T, W);
  if (wf == wl) return;  // whole sequence inside one range: already final
  const int first_which = s0 == range_start(wf, T, W) ? 0 : 1;
  constexpr int LPH = D / 4;      // lanes per head row
  constexpr int HPI = 64 / LPH;   // heads per iteration
  const int hl = lane / LPH;
  const int d4 = (lane % LPH) * 4;
  for (int h0 = 0; h0 < P.group; h0 += HPI) {
    const int h = h0 + hl;
    if (h >= P.group) continue;
    // wavefronts with an empty range (more wavefronts than blocks) hold no piece
    float M = -INFINITY;
    for (int64_t wv = wf; wv <= wl; ++wv) {
      if (range_start(wv + 1, T, W) == range_start(wv, T, W)) continue;
      const int which = wv == wf ? first_which : 0;
      M = fmaxf(M, P.ws_ml[((wv * 2 + which) * P.group + h) * 2]);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float Lsum = 0.f;
    if (M != -INFINITY) {
      for (int64_t wv = wf; wv <= wl; ++wv) {
        if (range_start(wv + 1, T, W) == range_start(wv, T, W)) continue;
        const int which = wv == wf ? first_which : 0;
        const int64_t slot = (wv * 2 + which) * P.group + h;
        const f32x2 ml = *reinterpret_cast<const f32x2*>(P.ws_ml + slot * 2);
        const float wt = __builtin_amdgcn_exp2f(ml[0] - M);
        Lsum += wt * ml[1];
        acc += wt * *reinterpret_cast<const f32x4*>(P.ws_o + slot * D + d4);
      }
    }
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    const int64_t off = ((int64_t)b * P.hq + (int64_t)g * P.group + h) * D + d4;
    const f32x4 o = acc * inv;
    if (P.out_dtype == PKV_F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.out) + off) = o;
    } else if (P.out_dtype == PKV_BF16) {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + off) =
          make_uint2(f32_to_bf16_bits_rne(o[0]) | (f32_to_bf16_bits_rne(o[1]) << 16),
                     f32_to_bf16_bits_rne(o[2]) | (f32_to_bf16_bits_rne(o[3]) << 16));
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + off) =
          make_uint2(f32_to_f16_bits(o[0]) | (f32_to_f16_bits(o[1]) << 16),
                     f32_to_f16_bits(o[2]) | (f32_to_f16_bits(o[3]) << 16));
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static constexpr int kWavesPerCU = 8;
static constexpr int kMaxBatch = 16000;   // C[] of B+1 ints in LDS

static pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static pkv_status device_cus(int* cus) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (!cache[dev]) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    cache[dev] = n;
  }
  *cus = cache[dev];
  return PKV_OK;
}

static bool supported_shape(int d, int bs) {
  return (d == 64 || d == 128) && (bs == 16 || bs == 32 || bs == 64 || bs == 128);
}

static int expected_q_dtype(int kv) { return kv == PKV_FP8_E4M3 ? PKV_BF16 : kv; }

static pkv_status check_decode(const kv_pool* pool, const paged_decode_args* a) {
  if (!pool || !a) return fail(PKV_E_INVAL, "null argument");
  const kv_pool_desc& d = pool->desc;
  if (!d.k_cache || !d.v_cache) return fail(PKV_E_INVAL, "pool has no device buffers");
  if (!supported_shape(d.head_dim, d.block_size))
    return fail(PKV_E_UNSUPPORTED, "head_dim must be 64 or 128 and block_size 16, 32, 64 or 128");
  if (a->layer < 0 || a->layer >= d.num_layers) return fail(PKV_E_INVAL, "layer out of range");
  if (a->batch < 0) return fail(PKV_E_INVAL, "batch must be >= 0");
  if (a->batch > kMaxBatch) return fail(PKV_E_UNSUPPORTED, "batch above 16000");
  if (a->num_q_heads <= 0 || a->num_q_heads % d.num_kv_heads)
    return fail(PKV_E_INVAL, "num_q_heads must be a positive multiple of num_kv_heads");
  if (a->num_q_heads / d.num_kv_heads > 16) return fail(PKV_E_UNSUPPORTED, "query group above 16");
  if (a->max_blocks_per_seq < 0 || a->sliding_window < 0 || a->num_splits < 0)
    return fail(PKV_E_INVAL, "negative max_blocks_per_seq, sliding_window or num_splits");
  if (a->q_dtype != expected_q_dtype(d.kv_dtype))
    return fail(PKV_E_DTYPE, "q_dtype must be f32 / f16 / bf16 for f32 / f16 / (bf16, fp8) pools");
  if (a->out_dtype != PKV_F32 && a->out_dtype != PKV_F16 && a->out_dtype != PKV_BF16)
    return fail(PKV_E_DTYPE, "out_dtype must be f32, f16 or bf16");
  if (!std::isfinite(a->scale)) return fail(PKV_E_INVAL, "scale must be finite");
  if (a->batch > 0 && (!a->q || !a->out || !a->context_lens || (a->max_blocks_per_seq > 0 && !a->block_tables)))
    return fail(PKV_E_INVAL, "null device pointer");
  return PKV_OK;
}

static int64_t num_waves_for(const paged_decode_args* a, int cus) {
  return a->num_splits >= 2 ? (int64_t)a->num_splits : (int64_t)cus * kWavesPerCU;
}

static size_t workspace_for(const kv_pool* pool, const paged_decode_args* a, int64_t W) {
  const int64_t G = a->num_q_heads / pool->desc.num_kv_heads;
  const size_t o = (size_t)W * 2 * G * pool->desc.head_dim * sizeof(float);
  const size_t ml = (size_t)W * 2 * G * 2 * sizeof(float);
  return ((o + 255) / 256) * 256 + ml;
}

typedef void (*decode_fn)(DecodeParams);

template <int KV, int D>
static decode_fn pick_decode_bs(int bs) {
  switch (bs) {
    case 16: return decode_kernel<KV, D, 16>;
    case 32: return decode_kernel<KV, D, 32>;
    case 64: return decode_kernel<KV, D, 64>;
    case 128: return decode_kernel<KV, D, 128>;
  }
  return nullptr;
}

template <int KV>
static decode_fn pick_decode_d(int d, int bs) {
  return d == 64 ? pick_decode_bs<KV, 64>(bs) : pick_decode_bs<KV, 128>(bs);
}

static decode_fn pick_decode(int kv, int d, int bs) {
  switch (kv) {
    case PKV_F32: return pick_decode_d<KV_F32>(d, bs);
    case PKV_F16: return pick_decode_d<KV_F16>(d, bs);
    case PKV_BF16: return pick_decode_d<KV_BF16>(d, bs);
    case PKV_FP8_E4M3: return pick_decode_d<KV_FP8>(d, bs);
  }
  return nullptr;
}

template <int D>
static decode_fn pick_merge_bs(int bs) {
  switch (bs) {
    case 16: return merge_kernel<D, 16>;
    case 32: return merge_kernel<D, 32>;
    case 64: return merge_kernel<D, 64>;
    case 128: return merge_kernel<D, 128>;
  }
  return nullptr;
}

static decode_fn pick_merge(int d, int bs) { return d == 64 ? pick_merge_bs<64>(bs) : pick_merge_bs<128>(bs); }

}  // namespace pkv

using namespace pkv;

extern "C" {

pkv_status kv_pool_copy_blocks(kv_pool* pool, const kv_block_copy* d_pairs, int32_t n, pkv_stream stream) {
  if (!pool || n < 0 || (n > 0 && !d_pairs)) return fail(PKV_E_INVAL, "bad argument");
  const kv_pool_desc& d = pool->desc;
  if (!d.k_cache || !d.v_cache) return fail(PKV_E_INVAL, "pool has no device buffers");
  if (n == 0) return PKV_OK;
  const int64_t tile_bytes = (int64_t)d.num_kv_heads * d.block_size * d.head_dim * elem_bytes(d.kv_dtype);
  if (tile_bytes % 16) return fail(PKV_E_UNSUPPORTED, "block bytes must be a multiple of 16");
  dim3 grid(n, d.num_layers, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)d.k_cache, (uint8_t*)d.v_cache, d_pairs, (int64_t)d.num_blocks, tile_bytes);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : hip_fail(e, "copy_blocks launch");
}

pkv_status paged_kv_append(kv_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                           int32_t src_dtype, const int64_t* d_slots, int32_t n_tokens,
                           pkv_stream stream) {
  if (!pool || n_tokens < 0) return fail(PKV_E_INVAL, "bad argument");
  const kv_pool_desc& d = pool->desc;
  if (!d.k_cache || !d.v_cache) return fail(PKV_E_INVAL, "pool has no device buffers");
  if (layer < 0 || layer >= d.num_layers) return fail(PKV_E_INVAL, "layer out of range");
  if (!supported_shape(d.head_dim, d.block_size))
    return fail(PKV_E_UNSUPPORTED, "head_dim must be 64 or 128 and block_size 16, 32, 64 or 128");
  const bool same = src_dtype == d.kv_dtype;
  const bool quant = d.kv_dtype == PKV_FP8_E4M3 &&
                     (src_dtype == PKV_F32 || src_dtype == PKV_F16 || src_dtype == PKV_BF16);
  if (!same && !quant) return fail(PKV_E_DTYPE, "unsupported source dtype for this pool");
  if (n_tokens == 0) return PKV_OK;
  if (!d_k || !d_v || !d_slots) return fail(PKV_E_INVAL, "null device pointer");
  AppendParams P;
  P.kc = (uint8_t*)d.k_cache;
  P.vc = (uint8_t*)d.v_cache;
  P.k = (const uint8_t*)d_k;
  P.v = (const uint8_t*)d_v;
  P.slots = d_slots;
  P.k_inv = d.k_inv_scale;
  P.v_inv = d.v_inv_scale;
  P.num_blocks = d.num_blocks;
  P.n = n_tokens;
  P.hkv = d.num_kv_heads;
  P.d = d.head_dim;
  P.bs = d.block_size;
  P.layer = layer;
  const int X = 16 / elem_bytes(d.kv_dtype);
  const int64_t total = (int64_t)n_tokens * d.num_kv_heads * (d.head_dim / X);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return fail(PKV_E_UNSUPPORTED, "too many tokens in one append");
  void (*fn)(AppendParams) = nullptr;
  if (same) {
    switch (d.kv_dtype) {
      case PKV_F32: fn = append_kernel<KV_F32, KV_F32>; break;
      case PKV_F16: fn = append_kernel<KV_F16, KV_F16>; break;
      case PKV_BF16: fn = append_kernel<KV_BF16, KV_BF16>; break;
      default: break;
    }
  } else {
    switch (src_dtype) {
      case PKV_F32: fn = append_kernel<KV_FP8, KV_F32>; break;
      case PKV_F16: fn = append_kernel<KV_FP8, KV_F16>; break;
      case PKV_BF16: fn = append_kernel<KV_FP8, KV_BF16>; break;
      default: break;
    }
  }
  if (!fn) return fail(PKV_E_DTYPE, "unsupported dtype combination");
  hipLaunchKernelGGL(fn, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream, P);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : hip_fail(e, "append launch");
}

pkv_status paged_attention_workspace_size(const kv_pool* pool, const paged_decode_args* a, size_t* bytes_out) {
  if (!bytes_out) return fail(PKV_E_INVAL, "null argument");
  pkv_status st = check_decode(pool, a);
  if (st != PKV_OK) return st;
  if (a->num_splits == 1) {
    *bytes_out = 0;
    return PKV_OK;
  }
  int cus = 0;
  if (a->num_splits == 0) {
    st = device_cus(&cus);
    if (st != PKV_OK) return st;
  }
  *bytes_out = workspace_for(pool, a, num_waves_for(a, cus));
  return PKV_OK;
}

pkv_status paged_attention_decode(const kv_pool* pool, const paged_decode_args* a, pkv_stream stream) {
  pkv_status st = check_decode(pool, a);
  if (st != PKV_OK) return st;
  if (a->batch == 0) return PKV_OK;
  const kv_pool_desc& d = pool->desc;
  DecodeParams P;
  P.kc = (const uint8_t*)d.k_cache;
  P.vc = (const uint8_t*)d.v_cache;
  P.k_scale = d.k_scale;
  P.v_scale = d.v_scale;
  P.q = (const uint8_t*)a->q;
  P.out = (uint8_t*)a->out;
  P.tables = a->block_tables;
  P.lens = a->context_lens;
  P.num_blocks = d.num_blocks;
  P.layer = a->layer;
  P.batch = a->batch;
  P.hq = a->num_q_heads;
  P.hkv = d.num_kv_heads;
  P.group = a->num_q_heads / d.num_kv_heads;
  P.max_blocks = a->max_blocks_per_seq;
  P.window = a->sliding_window;
  P.out_dtype = a->out_dtype;
  P.scale_log2 = a->scale * 1.4426950408889634f;
  P.ws_o = nullptr;
  P.ws_ml = nullptr;
  P.xcd_remap = 0;
  decode_fn fn = pick_decode(d.kv_dtype, d.head_dim, d.block_size);
  if (!fn) return fail(PKV_E_UNSUPPORTED, "no kernel for this shape");
  hipStream_t s = (hipStream_t)stream;
  const int64_t segs = (int64_t)d.num_kv_heads * a->batch;

  if (a->num_splits == 1 || a->max_blocks_per_seq == 0) {
    P.single = 1;
    P.num_waves = 0;
    const int64_t grid = (segs + 3) / 4;
    hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(256), 0, s, P);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PKV_OK : hip_fail(e, "decode launch");
  }

  int cus = 0;
  if (a->num_splits == 0) {
    st = device_cus(&cus);
    if (st != PKV_OK) return st;
  }
  const int64_t W = num_waves_for(a, cus);
  if (W > INT32_MAX / 2) return fail(PKV_E_INVAL, "num_splits too large");
  const size_t need = workspace_for(pool, a, W);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(PKV_E_INVAL, "workspace missing or smaller than paged_attention_workspace_size()");
  if (reinterpret_cast<uintptr_t>(a->workspace) % 256) return fail(PKV_E_INVAL, "workspace must be 256-byte aligned");
  const int64_t G = P.group;
  P.ws_o = reinterpret_cast<float*>(a->workspace);
  const size_t o_bytes = (size_t)W * 2 * G * d.head_dim * sizeof(float);
  P.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(a->workspace) + ((o_bytes + 255) / 256) * 256);
  P.single = 0;
  P.num_waves = (int32_t)W;
  const int64_t grid = (W + 3) / 4;
  P.xcd_remap = grid % 8 == 0 ? 1 : 0;
  const size_t lds = (size_t)(a->batch + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(fn, dim3((uint32_t)grid), dim3(256), lds, s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  decode_fn mfn = pick_merge(d.head_dim, d.block_size);
  const int64_t mgrid = (segs + 3) / 4;
  hipLaunchKernelGGL(mfn, dim3((uint32_t)mgrid), dim3(256), lds, s, P);
  e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : hip_fail(e, "merge launch");
}

}  // extern "C"
