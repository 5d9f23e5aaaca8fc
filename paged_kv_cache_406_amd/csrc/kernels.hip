// Device side of the paged KV-cache library for gfx950 (CDNA4).
//
// Kernels
//   append_kernel      new tokens' K/V into their slots (bit copy, or FP8
//                      quantise-on-write with per-channel inverse scales)
//   copy_blocks_kernel whole-block copies for copy-on-write
//   decode_kernel      decode attention over the paged cache: per-wavefront
//                      ranges of (KV head, sequence, work unit), QK^T and PV
//                      on MFMA, online softmax in registers; sequences whose
//                      units straddle ranges leave partial results
//   merge_kernel       log-sum-exp merge of those partial results
//   upload_kernel      per-step metadata from page-locked host memory
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
//    wavefront owns a (KV head, sequence, unit range).  A sub-tile of 16
//    (fp32), 32 (fp16 / bf16) or 64 (FP8) tokens of K and V goes from HBM
//    straight into MFMA operand registers with 16-byte loads in every lane
//    and is used for all G query heads of the group at once (the GQA reuse);
//    the next sub-tile's loads are issued before the current one is scored
//    (two register buffers).
//  * QK^T: S_t[16 tokens][16 heads] = K_t[16 tokens][D] * Q^T[D][16 heads] on
//    v_mfma_f32_16x16x32 (bf16 / f16; FP8 codes widened exactly to bf16) or
//    16x16x4 (f32).  Query heads beyond G are zero columns.  The rows of the
//    QK tiles are assigned to tokens so that every lane ends up holding the
//    scores of exactly the 8 (16) consecutive tokens whose V it loaded, which
//    is the B operand of PV: P never moves between lanes.
//  * PV: O^T[16 dims][16 heads] += V^T[16 dims][32 tokens] * P^T[32 tokens][16 heads].
//    V is stored channel-major inside a block so that a lane's tokens of one
//    channel are contiguous.  bf16 P is split into hi + lo bf16 parts (two
//    MFMAs) so the rounding of P stays far below fp32 accumulation error.
//  * The max of each head's scores is shared by the 4 lanes holding that head
//    (two lane exchanges); sums stay per lane until the end.
//  * Work split: the sub-tile-aligned units of all (KV head, sequence) pairs
//    are laid end to end (KV-head major) and cut into W equal ranges, one per
//    wavefront.  A wavefront streams its range as one sequence of sub-tiles,
//    its loads one sub-tile ahead across the boundaries between sequences.
//    A range that covers a whole sequence writes the final output; a piece
//    of a sequence that straddles ranges is written as (unnormalised o, max,
//    sum), and merge_kernel combines the pieces.  Workgroups are remapped so
//    that each XCD (one L2) gets a contiguous run of ranges.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "pool_internal.h"

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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

// Tokens per sub-tile: the amount one wavefront loads and scores at a time.
// Each lane group (16 lanes) holds TT/4 consecutive tokens of V, which is
// 16 bytes for every element size.
template <int KV> struct SubTile;
template <> struct SubTile<KV_F32> { static constexpr int TT = 16; };
template <> struct SubTile<KV_F16> { static constexpr int TT = 32; };
template <> struct SubTile<KV_BF16> { static constexpr int TT = 32; };
template <> struct SubTile<KV_FP8> { static constexpr int TT = 64; };

// V inside a (block, KV head) tile: runs of VT = min(block size, TT)
// tokens, channel-major within a run, [bs / VT][D][VT].  At bs <= TT that is
// plain channel-major [D][bs]; for longer blocks each sub-tile's V is one
// contiguous D * TT run.
__host__ __device__ constexpr int v_run(int bs, int tt) { return bs < tt ? bs : tt; }

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
  // step mode (tables != NULL): token i is row i's next token; its block
  // goes into tables[i][lens[i] / bs] and lens[i] grows by one, and the slots
  // may be in page-locked host memory (read with system-scope loads)
  int32_t* tables;
  int32_t* lens;
  int32_t max_blocks;
};

// Raw bits of source element idx (fp32, or fp16 / bf16 in the low half).
template <int SRC>
__device__ __forceinline__ uint32_t src_bits(const uint8_t* p, int64_t idx) {
  if constexpr (SRC == KV_F32) return reinterpret_cast<const uint32_t*>(p)[idx];
  else return reinterpret_cast<const uint16_t*>(p)[idx];
}
template <int SRC>
__device__ __forceinline__ float bits_to_f32(uint32_t b) {
  if constexpr (SRC == KV_F32) return __uint_as_float(b);
  else if constexpr (SRC == KV_F16) return f16_bits_to_f32(b);
  else return bf16_bits_to_f32(b);
}

// What one thread stores of a token: its K group c (X channels, 16 bytes in
// the pool) and its X V elements (dims e * D/X + c) of one KV head, as raw
// source bits, with the channels' inverse scales for FP8.  Loading it is
// split from storing it so that every load is issued before the first
// store (the compiler may not move a load above a store that could alias
// it, so loads and stores taken in turn would cost one memory round trip
// per element), and before the slot is known.
template <int KV, int SRC>
struct TokenChunk {
  static constexpr int X = 16 / Elem<KV>::bytes;
  u32x4 k;                 // same dtype: the K group's bits
  uint32_t v[X];           // same dtype: the V elements' bits
  uint32_t kb[X], vb[X];   // FP8: source bits of the K channels and V elements
  float ki[X], vi[X];      // FP8: their inverse scales
};

// The loads of chunk c of KV head h from source row `row` (element index of
// the token's head row in k / v) of `layer`.
template <int KV, int SRC>
__device__ __forceinline__ TokenChunk<KV, SRC> load_token_chunk(const uint8_t* k, const uint8_t* v,
                                                                const float* k_inv, const float* v_inv, int hkv,
                                                                int d, int layer, int64_t row, int c, int h) {
  constexpr int X = TokenChunk<KV, SRC>::X;
  const int chunks = d / X;
  TokenChunk<KV, SRC> t;
  if constexpr (KV == SRC) {
    t.k = *reinterpret_cast<const u32x4*>(k + (row + (int64_t)c * X) * Elem<KV>::bytes);
#pragma unroll
    for (int e = 0; e < X; ++e) t.v[e] = src_bits<SRC>(v, row + (int64_t)e * chunks + c);
  } else {
    static_assert(KV == KV_FP8, "only same-dtype copy or FP8 quantisation");
    const int64_t s0 = ((int64_t)layer * hkv + h) * d;   // channel scales of (layer, head)
#pragma unroll
    for (int e = 0; e < X; ++e) {
      const int kd = c * X + e;
      const int64_t vd = (int64_t)e * chunks + c;
      t.kb[e] = src_bits<SRC>(k, row + kd);
      t.ki[e] = k_inv[s0 + kd];
      t.vb[e] = src_bits<SRC>(v, row + vd);
      t.vi[e] = v_inv[s0 + vd];
    }
  }
  return t;
}

// Store a loaded chunk into block blk at offset off of `layer`: a bit copy,
// or the E4M3 codes of x * inv_scale.
template <int KV, int SRC>
__device__ __forceinline__ void store_token_chunk(const TokenChunk<KV, SRC>& t, uint8_t* kc, uint8_t* vc,
                                                  int64_t num_blocks, int hkv, int d, int bs, int layer, int c,
                                                  int h, int64_t blk, int off) {
  constexpr int EB = Elem<KV>::bytes;
  constexpr int X = TokenChunk<KV, SRC>::X;
  const int chunks = d / X;
  const int64_t tile = ((int64_t)layer * num_blocks + blk) * hkv + h;
  uint8_t* kdst = kc + ((tile * (d / X) + c) * bs + off) * 16;
  // V runs of vt tokens, channel-major inside a run: element dim of this
  // token sits vt elements after element dim - 1.  The thread's e-th V
  // element is dim e * chunks + c, so the lanes of one store instruction
  // cover consecutive dims, and the dims that share a cache line are written
  // by one instruction.
  const int vt = v_run(bs, SubTile<KV>::TT);
  uint8_t* vdst = vc + (tile * d * bs + (int64_t)(off / vt) * d * vt + off % vt) * EB;
  // non-temporal stores: the cache lines this token touches (one 16-byte K
  // group, D V elements in bs-element rows) are not read again by this kernel
  if constexpr (KV == SRC) {
    __builtin_nontemporal_store(t.k, reinterpret_cast<u32x4*>(kdst));
#pragma unroll
    for (int e = 0; e < X; ++e) {
      uint8_t* dst = vdst + ((int64_t)e * chunks + c) * vt * EB;
      if constexpr (EB == 4)
        __builtin_nontemporal_store(t.v[e], reinterpret_cast<uint32_t*>(dst));
      else
        __builtin_nontemporal_store((uint16_t)t.v[e], reinterpret_cast<uint16_t*>(dst));
    }
  } else {
    uint32_t kw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < X; ++e) {
      kw[e >> 2] |= f32_to_e4m3(bits_to_f32<SRC>(t.kb[e]) * t.ki[e]) << (8 * (e & 3));
      __builtin_nontemporal_store((uint8_t)f32_to_e4m3(bits_to_f32<SRC>(t.vb[e]) * t.vi[e]),
                                  vdst + ((int64_t)e * chunks + c) * vt);
    }
    __builtin_nontemporal_store(u32x4{kw[0], kw[1], kw[2], kw[3]}, reinterpret_cast<u32x4*>(kdst));
  }
}

template <int KV, int SRC>
__global__ __launch_bounds__(256) void append_kernel(AppendParams P) {
  constexpr int X = 16 / Elem<KV>::bytes;
  const int chunks = P.d / X;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)P.n * P.hkv * chunks;
  const int64_t per_row = (int64_t)chunks * P.hkv;
  const int c = (int)(t % chunks);
  const int h = (int)((t / chunks) % P.hkv);
  const int64_t i = t / per_row;
  // The threads of one token are consecutive: the first lane of each token
  // in the wavefront reads its slot (from page-locked host memory, one
  // transfer per token rather than one per thread) and the others take it
  // from that lane.  The source lane is never past the reading lane, so it
  // is active whenever the reading lane is.
  const int lane = (int)(threadIdx.x & 63);
  const int64_t pos = t - i * per_row;
  const int src = pos <= lane ? lane - (int)pos : 0;
  // this thread's chunk, loaded before its slot is known (lanes past the end
  // load the last chunk, so that no branch sits around the loads)
  const int64_t tl = t < total ? t : total - 1;
  const int hl = (int)((tl / chunks) % P.hkv);
  const TokenChunk<KV, SRC> tok = load_token_chunk<KV, SRC>(P.k, P.v, P.k_inv, P.v_inv, P.hkv, P.d, P.layer,
                                                            ((tl / per_row) * P.hkv + hl) * P.d,
                                                            (int)(tl % chunks), hl);
  int64_t slot = -1;
  if (t < total && lane == src)
    slot = P.tables ? __hip_atomic_load(P.slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : P.slots[i];
  slot = __shfl(slot, src);
  if (t >= total) return;
  if (slot < 0 || slot >= P.num_blocks * P.bs) return;
  const int64_t blk = slot / P.bs;
  const int off = (int)(slot % P.bs);
  if (P.tables && h == 0 && c == 0) {
    // the row's table and length follow the host block manager's decision,
    // which the slot encodes: block slot / bs at position lens[i]
    const int32_t pos = P.lens[i];
    if (pos >= 0 && pos / P.bs < P.max_blocks) {
      P.tables[i * P.max_blocks + pos / P.bs] = (int32_t)blk;
      P.lens[i] = pos + 1;
    }
  }
  store_token_chunk<KV, SRC>(tok, P.kc, P.vc, P.num_blocks, P.hkv, P.d, P.bs, P.layer, c, h, blk, off);
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
  const u32x4* s = reinterpret_cast<const u32x4*>(base + ((int64_t)layer * num_blocks + src) * tile_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + ((int64_t)layer * num_blocks + dst) * tile_bytes);
  const int64_t n16 = tile_bytes / 16;
  // Streamed: neither copy is read again by this kernel, and dirty lines
  // left in L2 would be written back while the next kernel runs.  Each
  // thread loads a batch of 16-byte groups before storing any of them: the
  // source and destination blocks differ, but the compiler cannot know that
  // and would otherwise wait for every load before the store after it.
  constexpr int BATCH = 8;
  const int64_t bd = blockDim.x;
  int64_t i0 = threadIdx.x;
  for (; i0 + (BATCH - 1) * bd < n16; i0 += BATCH * bd) {
    u32x4 v[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) v[k] = __builtin_nontemporal_load(s + i0 + k * bd);
#pragma unroll
    for (int k = 0; k < BATCH; ++k) __builtin_nontemporal_store(v[k], d + i0 + k * bd);
  }
  for (; i0 < n16; i0 += bd) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i0), d + i0);
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

struct DecodeParams {
  const uint8_t* kc;
  const uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* q;
  uint8_t* out;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_o;        // [W][2][G][D] unnormalised partial outputs
  float* ws_ml;       // [W][2][G][2] partial (max, sum), log2 domain
  int4* ws_job;       // [Hkv][B] merge job of each (KV head, sequence): {first range,
                      // pieces, slot of the first piece, 0}; pieces = 0: nothing to merge
  int64_t num_blocks;
  int32_t layer, batch, hq, hkv, group, max_blocks, window, out_dtype;
  int32_t num_waves;  // W: wavefront ranges (range mode)
  int32_t single;     // 1: one wavefront per (KV head, sequence)
  int32_t xcd_remap;
  float scale_log2;   // scale * log2(e)
  // shared prefix: the first `shared` table entries of every row are row 0's
  // blocks; prefix_kernel leaves one partial (o[D], max, sum) per (chunk,
  // sequence, query head) in ws_pre, and merge_kernel folds them in
  int32_t shared;     // 0: off
  int32_t pre_chunks; // token chunks of the prefix
  int32_t pre_rtiles; // query-row groups (one workgroup each) per KV head
  float* ws_pre;      // [pre_chunks + 1][B * Hq][D + 4]: o, max, sum, 2 pad
  // range mode: results of pieces that end before a wavefront's range does
  // are kept in LDS (up to `nstage` per wavefront, from byte `stage_off` of
  // the dynamic LDS block) and written when the range is done
  int32_t nstage;
  int32_t stage_off;
  // range mode: 1 when the context lengths are also kept in LDS, after the
  // unit prefix sums (a piece's start then reads no global memory)
  int32_t lens_in_lds;
  // every (KV head, sequence) pair leaves a partial (o, max, sum) for
  // merge_kernel, also when one wavefront held all of it: with a shared
  // prefix, and with a fused append
  int32_t allpart;
  // fused append (fused = 1): lens[b] counts the cached tokens before the new
  // one.  The decode attends the cached tokens (the window counted over all
  // L + 1); merge_kernel folds in the new token as one more partial (scores
  // from new_k, values from new_v, quantised like the pool for FP8), writes
  // it into the pool at new_slots[b], writes the row's table entry and
  // lens[b] = L + 1.  A slot outside the pool is attended but not stored.
  int32_t fused;
  int32_t new_src;         // dtype of new_k / new_v
  int32_t kv_dtype;        // the pool's
  int32_t block_size;
  const uint8_t* new_k;    // [B][Hkv][D]
  const uint8_t* new_v;
  const int64_t* new_slots;  // [B], device or page-locked host memory
  const float* k_inv;      // FP8: inverse scales used to encode
  const float* v_inv;
  int32_t* tables_w;       // the same tables and lengths, written by merge_kernel
  int32_t* lens_w;
  int32_t merge_pg;        // merge workgroups per (KV head, sequence)
  int32_t append_spg;      // fused append: sequences per append workgroup
};

// Fused append, pools other than FP8: decode_kernel's workgroups past the
// first decode_wgs store the new tokens and copy each row's slot to ws_slots
// [B] (workspace); merge_kernel then writes the rows' table entries and
// lengths.  A kernel argument of its own, so that DecodeParams, and the code
// built for kernels that do not read these, stays as it is.
struct TailParams {
  int64_t* ws_slots;
  int32_t decode_wgs;
};

// Which piece an LDS staging slot of the decode holds (48 bytes, so that
// slots and wavefront areas stay 16-byte aligned).
struct PieceTag {
  int32_t g, b, nb, pad;
  int64_t start, beg, end, pad2;
};
static_assert(sizeof(PieceTag) == 48, "staging tag layout");


template <int KV, int BS>
struct Units {
  static constexpr int TT = SubTile<KV>::TT;
  static constexpr int U = BS > TT ? BS : TT;  // tokens per work unit (whole blocks, whole sub-tiles)
  static constexpr int UB = U / BS;            // blocks per unit
};

// Attended range of sequence b: L tokens (clamped to the table), first key
// lo (window), first block, and the number of work units from that block on.
template <int BS, int U>
__device__ __forceinline__ void extent_of(const DecodeParams& P, int32_t L, int32_t* L_out, int32_t* lo_out,
                                          int32_t* first_out, int32_t* nunits_out) {
  const int32_t cap = P.max_blocks * BS;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  // with a fused append the window ends at the new token, one past L
  const int32_t Lw = L + (P.fused ? 1 : 0);
  const int32_t lo = P.window > 0 ? (Lw - P.window > 0 ? Lw - P.window : 0) : 0;
  // with a shared prefix (no window) the blocks before `shared` are
  // prefix_kernel's
  const int32_t first = P.shared > 0 ? P.shared : lo / BS;
  *L_out = L;
  *lo_out = lo;
  *first_out = first;
  *nunits_out = L > lo && L > first * BS ? (L - first * BS + U - 1) / U : 0;
}

template <int BS, int U>
__device__ __forceinline__ void seq_extent(const DecodeParams& P, int b, int32_t* L_out, int32_t* lo_out,
                                           int32_t* first_out, int32_t* nunits_out) {
  extent_of<BS, U>(P, P.lens[b], L_out, lo_out, first_out, nunits_out);
}

// Exclusive prefix sums of the per-sequence unit counts into C[0..B] (LDS);
// with lens_in_lds the context lengths follow, at C[B + 1 + b].
template <int BS, int U>
__device__ void scan_units(const DecodeParams& P, int32_t* C) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  const int per = (P.batch + 255) / 256;
  const int b0 = tid * per;
  const int b1 = min(P.batch, b0 + per);
  int32_t local = 0;
  for (int b = b0; b < b1; ++b) {
    const int32_t raw = P.lens[b];
    int32_t L, lo, first, nu;
    extent_of<BS, U>(P, raw, &L, &lo, &first, &nu);
    C[b] = nu;
    if (P.lens_in_lds) C[P.batch + 1 + b] = raw;
    local += nu;
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
    const int32_t nu = C[b];
    C[b] = run;
    run += nu;
  }
  if (tid == 255) C[P.batch] = part[255];
  __syncthreads();
}

// scan_units with the 256-wide scan done by lane exchanges inside each
// wavefront and one pass over the four wavefront totals: two barriers
// instead of sixteen.  Used by decode_append_kernel (decode_kernel keeps
// scan_units, see decode_body).
template <int BS, int U>
__device__ void scan_units_wave(const DecodeParams& P, int32_t* C) {
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int per = (P.batch + 255) / 256;
  const int b0 = tid * per;
  const int b1 = min(P.batch, b0 + per);
  int32_t local = 0;
  for (int b = b0; b < b1; ++b) {
    const int32_t raw = P.lens[b];
    int32_t L, lo, first, nu;
    extent_of<BS, U>(P, raw, &L, &lo, &first, &nu);
    C[b] = nu;
    if (P.lens_in_lds) C[P.batch + 1 + b] = raw;
    local += nu;
  }
  int32_t x = local;   // inclusive scan over the wavefront's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  int32_t before = 0;
  for (int k = 0; k < wv; ++k) before += wsum[k];
  const int32_t incl = before + x;
  int32_t run = incl - local;
  for (int b = b0; b < b1; ++b) {
    const int32_t nu = C[b];
    C[b] = run;
    run += nu;
  }
  if (tid == 255) C[P.batch] = incl;
  __syncthreads();
}

__device__ __forceinline__ int64_t range_start(int64_t w, int64_t T, int64_t W) { return w * T / W; }

// The wavefront whose range holds unit x (every range is non-empty: W <= T).
__device__ __forceinline__ int64_t wave_of(int64_t x, int64_t T, int64_t W) {
  return ((x + 1) * W - 1) / T;
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ void store4(const DecodeParams& P, int64_t off, const f32x4& o) {
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

template <int D>
__device__ __forceinline__ void write_zero_rows(const DecodeParams& P, int b, int g, int lane) {
  const int64_t row0 = ((int64_t)b * P.hq + (int64_t)g * P.group) * D;
  const int64_t n = (int64_t)P.group * D;
  for (int64_t e = lane; e < n; e += 64) {
    if (P.out_dtype == PKV_F32) reinterpret_cast<float*>(P.out)[row0 + e] = 0.f;
    else reinterpret_cast<uint16_t*>(P.out)[row0 + e] = 0;
  }
}

// 16-byte streaming load: the cache is read once per call, so K/V tiles
// are loaded non-temporally (no cache allocation for data that is not reused)
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane l's bytes land at LDS byte address
// lds_wave_base + 16 * l.  Written as inline assembly so that the compiler
// does not wait for these loads before every LDS read; the caller waits with
// wait_vmem and a barrier.  M0 (the LDS base) is set inside the same
// statement, right before the load.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds_wave_base), "v"(src) : "memory");
}

// Wait until at most N vector-memory loads of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  // gfx9 s_waitcnt: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14;
  // expcnt (bits 6:4) and lgkmcnt (bits 11:8) left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait_vmem<a * NG>() for a run-time a in [0, A] (a is wave-uniform).
template <int NG, int A>
__device__ __forceinline__ void wait_stages(int a) {
  if constexpr (A > 0) {
    if (a >= A) {
      wait_vmem<A * NG>();
      return;
    }
    wait_stages<NG, A - 1>(a);
  } else {
    wait_vmem<0>();
  }
}

// Entries rel .. rel + UB - 1 of a block-table row of n >= 1 entries (-1 from
// n on), read with scalar loads; rel is wave-uniform.  Scalar loads are
// counted by lgkmcnt, so waiting for them leaves the vector loads in flight
// alone (a vector load of a table entry inside a loop of untracked
// global-to-LDS loads makes the compiler wait for every load).  Each index
// is clamped into the row before it is read.
template <int UB>
__device__ __forceinline__ void table_entries_scalar(const int32_t* row, int32_t rel, int32_t n,
                                                     int32_t (&ids)[UB]) {
  static_assert(UB == 1 || UB == 2 || UB == 4, "blocks per unit");
  if (n <= 0) {
#pragma unroll
    for (int k = 0; k < UB; ++k) ids[k] = -1;
    return;
  }
  uint32_t off[UB];
#pragma unroll
  for (int k = 0; k < UB; ++k) off[k] = 4u * (uint32_t)(rel + k < n ? rel + k : n - 1);
  if constexpr (UB == 1) {
    asm volatile("s_load_dword %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=&s"(ids[0]) : "s"(row), "s"(off[0]) : "memory");
  } else if constexpr (UB == 2) {
    asm volatile("s_load_dword %0, %2, %3\n\ts_load_dword %1, %2, %4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(ids[0]), "=&s"(ids[1])
                 : "s"(row), "s"(off[0]), "s"(off[1])
                 : "memory");
  } else {
    asm volatile(
        "s_load_dword %0, %4, %5\n\ts_load_dword %1, %4, %6\n\ts_load_dword %2, %4, %7\n\t"
        "s_load_dword %3, %4, %8\n\ts_waitcnt lgkmcnt(0)"
        : "=&s"(ids[0]), "=&s"(ids[1]), "=&s"(ids[2]), "=&s"(ids[3])
        : "s"(row), "s"(off[0]), "s"(off[1]), "s"(off[2]), "s"(off[3])
        : "memory");
  }
#pragma unroll
  for (int k = 0; k < UB; ++k) ids[k] = rel + k < n ? ids[k] : -1;
}

// One wave-uniform int32 read with a scalar load (counted by lgkmcnt, not
// with the vector loads in flight).
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// LDS slots of the shared-prefix pipeline (16 KiB each); two workgroups of
// prefix_kernel share a CU
#ifndef PKV_PREFIX_STAGES
#define PKV_PREFIX_STAGES 3
#endif

// 16 bytes as 8 x 16-bit MFMA operand elements
template <typename V8>
__device__ __forceinline__ V8 as8(const uint4& w) {
  V8 r;
  __builtin_memcpy(&r, &w, 16);
  return r;
}

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t a, uint32_t b) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// One wavefront's view of the decode of a (KV head g, sequence b) piece.
//
// Lane l has i = l % 16 and kg = l / 16 (its lane group).  A sub-tile holds
// TT tokens; lane group kg owns the TPG = TT/4 consecutive tokens
// [TPG*kg, TPG*kg + TPG) of it.  Scores come from NQT = TT/16 MFMA tiles
// S_t[16 rows][16 heads]; row 4*kg + r of tile t is token TPG*kg + 4*t + r, so
// the output layout of S_t (lane (head, kg) holds rows 4*kg .. 4*kg+3) leaves
// every lane holding exactly the scores of its own lane group's tokens, which
// is the B operand the P.V MFMA needs, in the token order of its 16-byte V
// loads.  Query heads are MFMA columns (heads >= G are zero columns).
template <int KV, int D, int BS>
struct Decoder {
  static constexpr int EB = Elem<KV>::bytes;
  static constexpr int X = 16 / EB;                // channels per 16-byte K group
  static constexpr int TT = SubTile<KV>::TT;
  static constexpr int TPG = TT / 4;               // tokens per lane group
  static constexpr int NQT = TT / 16;              // QK tiles per sub-tile
  static constexpr int NKJ = D / (4 * X);          // K loads per lane per QK tile
  static constexpr int NKL = NQT * NKJ;            // K loads per lane per sub-tile
  static constexpr int NV = D / 16;                // V loads per lane per sub-tile = O tiles
  static constexpr int U = Units<KV, BS>::U;
  static constexpr int UB = Units<KV, BS>::UB;
  static constexpr int SPU = U / TT;               // sub-tiles per unit
  static constexpr int NQ = KV == KV_F32 ? D / 4 : D / 32;  // q operands per lane
  static constexpr int EPW = 4 / EB;               // V elements per dword
  static constexpr int64_t TILE_BYTES = (int64_t)D * BS * EB;  // one (block, KV head) tile
  static constexpr int VT = v_run(BS, TT);         // tokens per V run of a tile

  typedef typename std::conditional<KV == KV_F32, float,
          typename std::conditional<KV == KV_F16, f16x8, bf16x8>::type>::type qop;

  struct KTile {
    uint4 k[NKL];
  };
  struct VTile {
    uint4 v[NV];
    int32_t tok0;  // absolute index of the sub-tile's first token
    bool ok;       // this lane group's V block is a real block
  };
  // Where this lane's K rows and V tokens of one sub-tile live.
  struct Addr {
    const uint8_t* krow;  // this lane's first K group (channel group kg, its first row)
    const uint8_t* vrow;  // this lane's first V row (channel i, its first token)
    int32_t tok0;
    bool ok;
  };

  struct State {
    f32x4 O[NV];
    float m;
    float l;
  };

  // q operands of head i of group g.  Element e of operand s multiplies the
  // same channel as element e of the K operand of step s.  FP8 folds the
  // per-channel K scale into q (q'[c] = q[c] * k_scale[c]).  Lanes i >= G
  // (MFMA columns whose results are never written) read head 0's row.
  static __device__ __forceinline__ void load_q(const DecodeParams& P, int b, int g, int i, int kg,
                                                qop (&qo)[NQ]) {
    load_q_at(P, g, ((int64_t)b * P.hq + (int64_t)g * P.group + (i < P.group ? i : 0)) * D, kg, qo);
  }

  // Query row (element offset `row` of q, a head of KV head g) as this lane's
  // MFMA column.  The row must exist; the caller points the lanes of unused
  // columns at a real row.  Nothing is selected after the loads, so the wait
  // for them falls where the operands are first used, not here (the stream
  // prefetches the next piece's queries a sub-tile early).
  static __device__ __forceinline__ void load_q_at(const DecodeParams& P, int g, int64_t row, int kg,
                                                   qop (&qo)[NQ]) {
    if constexpr (KV == KV_F32) {
      const float* q = reinterpret_cast<const float*>(P.q) + row;
#pragma unroll
      for (int j = 0; j < NKJ; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) qo[4 * j + u] = q[(kg + 4 * j) * 4 + u];
    } else if constexpr (KV == KV_F16 || KV == KV_BF16) {
      const uint8_t* q = P.q + row * 2;
#pragma unroll
      for (int j = 0; j < NKJ; ++j) qo[j] = as8<qop>(*reinterpret_cast<const uint4*>(q + (kg + 4 * j) * 16));
    } else {
      const uint16_t* q = reinterpret_cast<const uint16_t*>(P.q) + row;
      const float* ks = P.k_scale + ((int64_t)P.layer * P.hkv + g) * D;
#pragma unroll
      for (int j = 0; j < NKJ; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int c = (kg + 4 * j) * 16 + 8 * h + e;
            const float x0 = bf16_bits_to_f32(q[c]) * ks[c];
            const float x1 = bf16_bits_to_f32(q[c + 1]) * ks[c + 1];
            w[e / 2] = f32_to_bf16_bits_rne(x0) | (f32_to_bf16_bits_rne(x1) << 16);
          }
          qo[2 * j + h] = as8<qop>(make_uint4(w[0], w[1], w[2], w[3]));
        }
    }
  }

  // Addresses of one sub-tile.  ids: the UB physical blocks of its unit
  // (uniform); st: sub-tile within the unit.  A lane whose block id is not a
  // real block reads block 0 instead and its tokens are masked later.
  static __device__ __forceinline__ Addr locate(const DecodeParams& P, int g, const int32_t (&ids)[UB], int st,
                                                int32_t tok0, int i, int kg) {
    int kb = 0, vb = 0, koff, voff;
    Addr a;
    if constexpr (UB == 1) {
      koff = st * TT + TPG * (i >> 2) + (i & 3);
      voff = st * TT + TPG * kg;
    } else {
      kb = (TPG * (i >> 2)) / BS;
      vb = (TPG * kg) / BS;
      koff = (TPG * (i >> 2)) % BS + (i & 3);
      voff = (TPG * kg) % BS;
    }
    int32_t pk = ids[0], pv = ids[0];
#pragma unroll
    for (int u = 1; u < UB; ++u) {
      pk = kb == u ? ids[u] : pk;
      pv = vb == u ? ids[u] : pv;
    }
    const bool okk = pk >= 0 && pk < P.num_blocks;
    const bool okv = pv >= 0 && pv < P.num_blocks;
    const int64_t head_tile = (int64_t)P.layer * P.num_blocks * P.hkv + g;
    a.krow = P.kc + (head_tile + (int64_t)(okk ? pk : 0) * P.hkv) * TILE_BYTES + (uint32_t)(kg * BS + koff) * 16u;
    // V: run voff / VT of the tile, channel i, token voff % VT of the run
    a.vrow = P.vc + (head_tile + (int64_t)(okv ? pv : 0) * P.hkv) * TILE_BYTES +
             (uint32_t)(((voff / VT) * D + i) * VT + voff % VT) * (uint32_t)EB;
    a.tok0 = tok0;
    a.ok = okv;
    return a;
  }

  // Constant offsets from the row pointers: K group kg + 4j and row + 4t;
  // V channel 16n + i.
  static __device__ __forceinline__ void load_k(KTile& T, const Addr& a) {
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int j = 0; j < NKJ; ++j)
        T.k[t * NKJ + j] = load_stream(a.krow + (4 * j * BS + 4 * t) * 16);
  }

  // Channel 16n + i of the run: VT elements after channel 16n + i - 1.  A
  // sub-tile's V is whole 128-byte lines (one run, or whole blocks), read
  // once: streamed.
  static __device__ __forceinline__ void load_v(VTile& T, const Addr& a) {
#pragma unroll
    for (int n = 0; n < NV; ++n) T.v[n] = load_stream(a.vrow + 16 * n * VT * EB);
    T.tok0 = a.tok0;
    T.ok = a.ok;
  }

  static __device__ __forceinline__ void qk(const KTile& T, const qop (&qo)[NQ], f32x4 (&S)[NQT]) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NKJ; ++j) {
        const uint4 w = T.k[t * NKJ + j];
        if constexpr (KV == KV_F32) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), qo[4 * j + 0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), qo[4 * j + 1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), qo[4 * j + 2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), qo[4 * j + 3], acc, 0, 0, 0);
        } else if constexpr (KV == KV_F16) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as8<f16x8>(w), qo[j], acc, 0, 0, 0);
        } else if constexpr (KV == KV_BF16) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as8<bf16x8>(w), qo[j], acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(w.x, w.y), qo[2 * j], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(w.z, w.w), qo[2 * j + 1], acc, 0, 0, 0);
        }
      }
      S[t] = acc;
    }
  }

  // Every lane's tokens of the sub-tile lie in a real block and in [lo, L),
  // so nothing needs masking (the same answer in every lane: a scalar
  // value, so the masked code below is branched around, not executed under
  // an exec mask).
  static __device__ __forceinline__ bool tile_full(const VTile& T, int32_t lo, int32_t L, int kg) {
    const int32_t t0 = T.tok0 + TPG * kg;
    return uniform((int)__all(T.ok && t0 >= lo && t0 + TPG <= L)) != 0;
  }

  // The exponentials of a (head, piece) are taken relative to a reference
  // maximum st.m that moves only when a score exceeds it by more than 2^8:
  // o and l are then at most 2^8 times larger than with the running maximum,
  // far from fp32 limits, and o / l -- like every use of (o, m, l) -- does not
  // depend on which reference was used.  So O is rescaled a few times per
  // piece instead of at every sub-tile.
  static constexpr float RESCALE_LOG2 = 8.0f;

  // Online softmax over one scored sub-tile: probabilities p of this lane's
  // tokens (0 where not attended), reference maximum, sum, O rescaled when
  // the reference moves.
  static __device__ __forceinline__ void softmax(const VTile& T, const f32x4 (&S)[NQT], State& st,
                                                 float (&p)[NQT][4], int32_t lo, int32_t L, float scale_log2,
                                                 int kg) {
    float s[NQT][4];
    if (tile_full(T, lo, L, kg)) {
#pragma unroll
      for (int t = 0; t < NQT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[t][r] = S[t][r] * scale_log2;
    } else {
      // The token base goes through an empty asm statement here, so that
      // the compares below cannot be hoisted above the branch into the
      // full-tile path (which would then run them on every sub-tile).
      int32_t base = T.tok0 + TPG * kg;
      asm volatile("" : "+v"(base));
#pragma unroll
      for (int t = 0; t < NQT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t tok = base + 4 * t + r;
          const bool valid = T.ok && tok >= lo && tok < L;
          s[t][r] = valid ? S[t][r] * scale_log2 : -INFINITY;
        }
    }
    float bmax = s[0][0];
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) bmax = fmaxf(bmax, s[t][r]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const bool up = bmax > st.m + RESCALE_LOG2;   // the first finite score always moves it
    if (__any(up)) {
      const float alpha = up ? __builtin_amdgcn_exp2f(st.m - bmax) : 1.0f;
      st.m = up ? bmax : st.m;
      st.l *= alpha;
#pragma unroll
      for (int n = 0; n < NV; ++n) st.O[n] *= alpha;
    }
    const float m_use = st.m == -INFINITY ? 0.f : st.m;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[t][r] = __builtin_amdgcn_exp2f(s[t][r] - m_use);
        psum += p[t][r];
      }
    st.l += psum;
  }

  // O += P.V over one sub-tile.  Tokens that are not attended may hold any
  // bits (NaN): their V elements are zeroed first (bit masks, no branch).
  static __device__ __forceinline__ void pv(VTile& T, const float (&p)[NQT][4], State& st, int32_t lo, int32_t L,
                                            int kg) {
    if (!tile_full(T, lo, L, kg)) {
      int32_t base = T.tok0 + TPG * kg;   // kept below the branch (see softmax)
      asm volatile("" : "+v"(base));
      mask_v(T, base, lo, L);
    }
    pv_acc(T, p, st);
  }

  // Zero the V elements of this lane's tokens base .. base + TPG - 1 that
  // are not attended (outside [lo, L), or not in a real block).
  static __device__ __forceinline__ void mask_v(VTile& T, int32_t base, int32_t lo, int32_t L) {
    uint32_t vmask[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < TPG; ++e) {
      const int32_t tok = base + e;
      const bool valid = T.ok && tok >= lo && tok < L;
      const uint32_t field = EB == 4 ? 0xffffffffu : (EB == 2 ? 0xffffu : 0xffu);
      vmask[e / EPW] |= valid ? field << (8 * EB * (e % EPW)) : 0u;
    }
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      T.v[n].x &= vmask[0];
      T.v[n].y &= vmask[1];
      T.v[n].z &= vmask[2];
      T.v[n].w &= vmask[3];
    }
  }

  // The MFMA part of pv: O += P.V with V already masked.
  static __device__ __forceinline__ void pv_acc(const VTile& T, const float (&p)[NQT][4], State& st) {
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        st.O[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(T.v[n].x), p[0][0], st.O[n], 0, 0, 0);
        st.O[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(T.v[n].y), p[0][1], st.O[n], 0, 0, 0);
        st.O[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(T.v[n].z), p[0][2], st.O[n], 0, 0, 0);
        st.O[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(T.v[n].w), p[0][3], st.O[n], 0, 0, 0);
      }
    } else if constexpr (KV == KV_F16) {
      f16x8 ph;
#pragma unroll
      for (int e = 0; e < 8; ++e) ph[e] = (_Float16)p[e / 4][e % 4];
#pragma unroll
      for (int n = 0; n < NV; ++n)
        st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as8<f16x8>(T.v[n]), ph, st.O[n], 0, 0, 0);
    } else {
      // P = hi + lo, both bf16 (hi = round(p), lo = round(p - hi)): the rounding
      // of P stays far below the fp32 accumulation error.
      constexpr int NC = TPG / 8;  // 32-token MFMA chunks per sub-tile
      bf16x8 phi[NC], plo[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f32x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = p[(8 * c + e) / 4][(8 * c + e) % 4];
        phi[c] = __builtin_convertvector(pf, bf16x8);
        plo[c] = __builtin_convertvector(pf - __builtin_convertvector(phi[c], f32x8), bf16x8);
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        if constexpr (KV == KV_BF16) {
          const bf16x8 a = as8<bf16x8>(T.v[n]);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi[0], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo[0], st.O[n], 0, 0, 0);
        } else {
          const bf16x8 a0 = e4m3x8_to_bf16x8(T.v[n].x, T.v[n].y);
          const bf16x8 a1 = e4m3x8_to_bf16x8(T.v[n].z, T.v[n].w);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, phi[0], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, plo[0], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, phi[1], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, plo[1], st.O[n], 0, 0, 0);
        }
      }
    }
  }

  // A (KV head, sequence) pair with keys to attend.  All fields uniform.
  struct Seg {
    int32_t g, b;
    int32_t L, lo, first;  // tokens, first attended key, its block
    int32_t nb;            // work units of the pair
    int64_t start;         // global index of the pair's first unit (range mode)
  };

  static __device__ __forceinline__ Seg make_seg(const DecodeParams& P, const int32_t* C, int64_t t_head, int g,
                                                 int b) {
    Seg s;
    int32_t nu;
    int32_t raw;
    if constexpr (KV != KV_FP8) {
      // Two loads of their own, each made uniform in its branch: written as
      // one select, they become a single generic (flat) load, which counts
      // as a vector load too, and waiting for it waits for every K/V load
      // in flight.
      if (C && P.lens_in_lds)
        raw = uniform(((const __attribute__((address_space(3))) int32_t*)C)[P.batch + 1 + b]);
      else
        raw = scalar_load_i32(P.lens + b);
    } else {
      raw = C && P.lens_in_lds ? C[P.batch + 1 + b] : P.lens[b];
    }
    extent_of<BS, U>(P, raw, &s.L, &s.lo, &s.first, &nu);
    s.g = g;
    s.b = b;
    s.L = uniform(s.L);
    s.lo = uniform(s.lo);
    s.first = uniform(s.first);
    if (C) {
      const int32_t cb = uniform(C[b]);
      s.nb = uniform(C[b + 1]) - cb;
      s.start = (int64_t)g * t_head + cb;
    } else {
      s.nb = uniform(nu);
      s.start = 0;
    }
    return s;
  }

  // The next pair after s that has units; false past the last KV head.
  static __device__ __forceinline__ bool next_seg(const DecodeParams& P, const int32_t* C, int64_t t_head,
                                                  const Seg& s, Seg& out) {
    int g = s.g, b = s.b;
    do {
      if (++b == P.batch) {
        b = 0;
        if (++g == P.hkv) return false;
      }
    } while (uniform(C[b + 1]) == uniform(C[b]));
    out = make_seg(P, C, t_head, g, b);
    return true;
  }

  // Entries [tb0 + 64c, tb0 + 64c + 64) of row b of the block tables, one
  // per lane (-1 from tb1 on).
  static __device__ __forceinline__ int32_t table_chunk(const DecodeParams& P, int b, int32_t tb0, int32_t tb1,
                                                        int c, int lane) {
    const int32_t idx = tb0 + 64 * c + lane;
    return idx < tb1 ? P.tables[(int64_t)b * P.max_blocks + idx] : -1;
  }

  // Units [beg, end) of pair s (global unit indices) -> its block-table range.
  static __device__ __forceinline__ void piece_blocks(const Seg& s, int64_t beg, int64_t end, int32_t* tb0,
                                                      int32_t* tb1) {
    const int32_t nblk = (s.L + BS - 1) / BS;
    *tb0 = s.first + (int32_t)(beg - s.start) * UB;
    *tb1 = min(s.first + (int32_t)(end - s.start) * UB, nblk);
  }

  // FP8: the per-channel V scale of this lane's output channels (1 otherwise).
  static __device__ __forceinline__ void v_scales(const DecodeParams& P, int g, int kg, float (&vsc)[NV][4]) {
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
  }

  // Row stride (floats) of a prefix partial: o[D], max, sum, 2 pad (16-byte rows).
  static constexpr int PRE_STRIDE = D + 4;

  // Final output or partial of the piece: units [beg, end) of pair s.  A
  // piece that is the whole pair writes the output rows; otherwise the
  // unnormalised o, max and sum go to workspace slot (w, which) for
  // merge_kernel, and the range holding the pair's first unit writes the
  // pair's merge job.
  static __device__ __forceinline__ void finish(const DecodeParams& P, const State& st, const Seg& s, int64_t beg,
                                                int64_t end, int64_t r0, int64_t T, int64_t W, int64_t w, int i,
                                                int kg, int lane) {
    const float l1 = st.l + __shfl_xor(st.l, 16);
    const float lall = l1 + __shfl_xor(l1, 32);
    // FP8: the per-channel V scale, applied once to the output
    float vsc[NV][4];
    v_scales(P, s.g, kg, vsc);
    const int G = P.group;
    const bool full = beg == s.start && end == s.start + s.nb;
    if (full && P.allpart) {
      // the whole of the pair's own part: its partial goes to the slot after
      // the prefix chunks, and merge_kernel joins the two (job.w = 1)
      if (lane == 0) P.ws_job[(int64_t)s.g * P.batch + s.b] = make_int4(0, 0, 0, 1);
      if (i >= G) return;
      const int64_t hrow = (int64_t)s.b * P.hq + (int64_t)s.g * G + i;
      float* base = P.ws_pre + ((int64_t)P.pre_chunks * P.batch * P.hq + hrow) * PRE_STRIDE;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = st.O[n][r] * vsc[n][r];
        *reinterpret_cast<f32x4*>(base + 16 * n + 4 * kg) = o;
      }
      if (kg == 0) *reinterpret_cast<f32x2*>(base + D) = f32x2{st.m, lall};
      return;
    }
    if (full) {
      if (!P.single && lane == 0) P.ws_job[(int64_t)s.g * P.batch + s.b] = make_int4(0, 0, 0, 0);
      if (i >= G) return;
      const float inv = lall > 0.f ? 1.0f / lall : 0.f;
      const int64_t row = ((int64_t)s.b * P.hq + (int64_t)s.g * G + i) * D;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = st.O[n][r] * inv * vsc[n][r];
        store4(P, row + 16 * n + 4 * kg, o);
      }
      return;
    }
    const int which = beg == r0 ? 0 : 1;
    if (beg == s.start && lane == 0) {
      const int64_t last = s.start + s.nb - 1;
      P.ws_job[(int64_t)s.g * P.batch + s.b] =
          make_int4((int)w, (int)(wave_of(last, T, W) - w + 1), which, 0);
    }
    if (i < G) {
      const int64_t slot = (w * 2 + which) * G + i;
      float* wo = P.ws_o + slot * D;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = st.O[n][r] * vsc[n][r];
        *reinterpret_cast<f32x4*>(wo + 16 * n + 4 * kg) = o;
      }
      if (kg == 0) *reinterpret_cast<f32x2*>(P.ws_ml + slot * 2) = f32x2{st.m, lall};
    }
  }

  // LDS staging of a finished piece.  A wavefront's area holds `nstage`
  // slots, then one PieceTag per slot.  Slot layout, npos = 4G positions
  // (lane (i, kg), i < G, at position kg * G + i): o as [NV][npos] 16-byte
  // groups (consecutive lanes 16 bytes apart), then (max, sum) as [npos].
  static __host__ __device__ constexpr int stage_slot_bytes(int G) { return 4 * G * (D + 8); }
  static __host__ __device__ constexpr int stage_area_bytes(int G, int nstage) {
    return nstage * (stage_slot_bytes(G) + (int)sizeof(PieceTag));
  }

  static __device__ __forceinline__ void stage_put(uint8_t* area, int nstage, int k, int G, const State& st,
                                                   const Seg& s, int64_t beg, int64_t end, int i, int kg,
                                                   int lane) {
    const int npos = 4 * G;
    uint8_t* slot = area + k * stage_slot_bytes(G);
    if (i < G) {
      const int pos = kg * G + i;
#pragma unroll
      for (int n = 0; n < NV; ++n) *reinterpret_cast<f32x4*>(slot + (n * npos + pos) * 16) = st.O[n];
      *reinterpret_cast<f32x2*>(slot + npos * D + pos * 8) = f32x2{st.m, st.l};
    }
    if (lane == 0) {
      PieceTag* t = reinterpret_cast<PieceTag*>(area + nstage * stage_slot_bytes(G)) + k;
      t->g = s.g;
      t->b = s.b;
      t->nb = s.nb;
      t->start = s.start;
      t->beg = beg;
      t->end = end;
    }
  }

  static __device__ __forceinline__ void stage_get(const uint8_t* area, int nstage, int k, int G, State& st,
                                                   Seg& s, int64_t* beg, int64_t* end, int i, int kg) {
    const int npos = 4 * G;
    const uint8_t* slot = area + k * stage_slot_bytes(G);
    const int pos = i < G ? kg * G + i : 0;
#pragma unroll
    for (int n = 0; n < NV; ++n) st.O[n] = *reinterpret_cast<const f32x4*>(slot + (n * npos + pos) * 16);
    const f32x2 ml = *reinterpret_cast<const f32x2*>(slot + npos * D + pos * 8);
    st.m = ml[0];
    st.l = ml[1];
    const PieceTag* t = reinterpret_cast<const PieceTag*>(area + nstage * stage_slot_bytes(G)) + k;
    s.g = uniform(t->g);
    s.b = uniform(t->b);
    s.nb = uniform(t->nb);
    s.start = uniform(t->start);
    s.L = s.lo = s.first = 0;
    *beg = uniform(t->beg);
    *end = uniform(t->end);
  }

  // Query-row tiles (MFMA column blocks of 16 rows) per wavefront of
  // prefix_kernel.  With one tile a wavefront needs at most 168 registers
  // (three per SIMD), so three workgroups share a CU; per query row the work
  // is the same as with two tiles, and the grid then needs fewer token
  // chunks.
  static constexpr int NT = 1;
  // 16-byte K and V groups of one sub-tile: one per lane per load of load_k /
  // load_v, so a wavefront's loads of a sub-tile are exactly the sub-tile.
  static constexpr int KG = NKL * 64;
  static constexpr int VG = NV * 64;
  // LDS bytes of one staged sub-tile (three are used)
  static constexpr int STAGE_BYTES = (KG + VG) * 16;
  static constexpr int STAGES = PKV_PREFIX_STAGES;

  // Maximum of v over the four lanes of a query row (lanes i, i + 16, i + 32,
  // i + 48): each swap leaves a lane's own value in one result and its
  // partner's (lane ^ 32, then lane ^ 16) in the other.
  static __device__ __forceinline__ float row_max4(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }

  // Online softmax of one row tile of the shared prefix (the decode's
  // softmax with the masking decided per sub-tile by the caller): with MASK,
  // tokens at or past the row's L, or in a block that is not real, get
  // probability 0.  scale_log2 >= 0 (the caller flips the sign of the
  // queries for a negative scale), so the row maximum of the scaled scores
  // is the scaled maximum of the raw ones, and each exponent is one fused
  // multiply-add.  Without MASK every score is finite.
  template <bool MASK>
  static __device__ __forceinline__ void prefix_softmax(const VTile& T, const f32x4 (&S)[NQT], State& st,
                                                        float (&p)[NQT][4], int32_t L, float scale_log2, int kg) {
    float s[NQT][4];
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (MASK) {
          const int32_t tok = T.tok0 + TPG * kg + 4 * t + r;
          s[t][r] = T.ok && tok < L ? S[t][r] * scale_log2 : -INFINITY;
        } else {
          s[t][r] = S[t][r];
        }
      }
    float bmax = s[0][0];
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) bmax = fmaxf(bmax, s[t][r]);
    bmax = row_max4(bmax);
    if constexpr (!MASK) bmax *= scale_log2;
    const bool up = bmax > st.m + RESCALE_LOG2;   // the first finite score always moves it
    if (__any(up)) {
      const float alpha = up ? __builtin_amdgcn_exp2f(st.m - bmax) : 1.0f;
      st.m = up ? bmax : st.m;
      st.l *= alpha;
#pragma unroll
      for (int n = 0; n < NV; ++n) st.O[n] *= alpha;
    }
    const float m_use = st.m == -INFINITY ? 0.f : st.m;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (MASK) {
          p[t][r] = __builtin_amdgcn_exp2f(s[t][r] - m_use);
        } else {
          p[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], scale_log2, -m_use));
        }
        psum += p[t][r];
      }
    st.l += psum;
  }

  // P = hi + lo for the P.V products of the shared prefix (16-bit-float
  // MFMA operands of bf16 and FP8 pools): hi = p rounded to bf16, lo = the
  // rest p - hi rounded to bf16, as the decode's P.V takes it; two values per
  // conversion, hi widened back with a shift and a mask.
  static __device__ __forceinline__ void split_p(const float (&p)[NQT][4], bf16x8 (&hi)[TPG / 8],
                                                 bf16x8 (&lo)[TPG / 8]) {
#pragma unroll
    for (int c = 0; c < TPG / 8; ++c) {
      u32x4 hw, lw;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 8 * c + 2 * k;
        const float a = p[e / 4][e % 4], b = p[(e + 1) / 4][(e + 1) % 4];
        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
        const f32x2 r = {a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u)};
        hw[k] = h;
        lw[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
      }
      hi[c] = __builtin_bit_cast(bf16x8, hw);
      lo[c] = __builtin_bit_cast(bf16x8, lw);
    }
  }

  // O += P.V of the shared prefix, V already masked.
  static __device__ __forceinline__ void prefix_pv(const VTile& T, const float (&p)[NQT][4], State& st) {
    if constexpr (KV == KV_F32 || KV == KV_F16) {
      pv_acc(T, p, st);
    } else {
      bf16x8 phi[TPG / 8], plo[TPG / 8];
      split_p(p, phi, plo);
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        if constexpr (KV == KV_BF16) {
          const bf16x8 a = as8<bf16x8>(T.v[n]);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi[0], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo[0], st.O[n], 0, 0, 0);
        } else {
          const bf16x8 a0 = e4m3x8_to_bf16x8(T.v[n].x, T.v[n].y);
          const bf16x8 a1 = e4m3x8_to_bf16x8(T.v[n].z, T.v[n].w);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, phi[0], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, plo[0], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, phi[1], st.O[n], 0, 0, 0);
          st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, plo[1], st.O[n], 0, 0, 0);
        }
      }
    }
  }

  // One staged sub-tile of the shared prefix for this wavefront's NT row
  // tiles: scores and softmax of each tile, then P.V of each.  Without MASK
  // every token is attended by every row.
  template <bool MASK>
  static __device__ __forceinline__ void prefix_step(const KTile& K, VTile& V, const qop (&q)[NT][NQ],
                                                     State (&st)[NT], const int32_t (&Lc)[NT], int32_t kT,
                                                     float scale_log2, int kg) {
    f32x4 S[NQT];
    float pp[NT][NQT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      qk(K, q[t], S);
      prefix_softmax<MASK>(V, S, st[t], pp[t], Lc[t], scale_log2, kg);
    }
    if constexpr (MASK) mask_v(V, V.tok0 + TPG * kg, 0, kT);
#pragma unroll
    for (int t = 0; t < NT; ++t) prefix_pv(V, pp[t], st[t]);
  }

  // Shared prefix, one workgroup of 4 wavefronts: query rows
  // rg*64*NT .. +64*NT of KV head g (wavefront wv takes 16*NT of them; row
  // r = sequence r / G, head g*G + r % G) against token chunk c of the prefix
  // (row 0's first `shared` blocks).  Every K/V sub-tile is fetched from
  // global memory once per workgroup, staged in LDS in the order in which a
  // wavefront's lanes use it, and read from there by all four wavefronts.
  // Each row attends the prefix tokens below min(its L, prefix).  Writes the
  // chunk's partial (o in output units, max, sum) of every row.
  static __device__ void prefix_group(const DecodeParams& P, int g, int rg, int c, uint8_t* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = lane & 15;
    const int kg = lane >> 4;
    const int wv = uniform(tid >> 6);
    const int G = P.group;
    const int64_t nrows = (int64_t)P.batch * G;
    const int32_t kT = P.shared * BS;
    const int32_t cap = P.max_blocks * BS;
    qop q[NT][NQ];
    State st[NT];
    int32_t Lc[NT];
    int64_t hrow[NT];
    bool live[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t r = ((int64_t)rg * 4 + wv) * 16 * NT + t * 16 + i;
      live[t] = r < nrows;
      const int b = live[t] ? (int)(r / G) : 0;
      const int hg = live[t] ? (int)(r % G) : 0;
      hrow[t] = (int64_t)b * P.hq + (int64_t)g * G + hg;
      load_q_at(P, g, hrow[t] * D, kg, q[t]);
      // a negative scale: flip the queries' signs (exact) and use |scale|
      if (P.scale_log2 < 0.f) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          if constexpr (KV == KV_F32)
            q[t][j] = -q[t][j];
          else
            q[t][j] = __builtin_bit_cast(qop, __builtin_bit_cast(u32x4, q[t][j]) ^ 0x80008000u);
        }
      }
      int32_t L = P.lens[b];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      Lc[t] = live[t] ? min(L, kT) : 0;
#pragma unroll
      for (int n = 0; n < NV; ++n) st[t].O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      st[t].m = -INFINITY;
      st[t].l = 0.f;
    }
    const int32_t nsp = (kT + TT - 1) / TT;
    const int32_t s0 = (int32_t)((int64_t)c * nsp / P.pre_chunks);
    const int32_t s1 = (int32_t)((int64_t)(c + 1) * nsp / P.pre_chunks);

    // the addresses this lane would load sub-tile s from (row 0's table
    // entries of the prefix, read with scalar loads)
    auto where = [&](int32_t s) -> Addr {
      const int32_t tok = s * TT;
      const int32_t rel = (tok / U) * UB;  // first table entry of the unit
      int32_t ids[UB];
      table_entries_scalar<UB>(P.tables, rel, P.shared, ids);
      return locate(P, g, ids, (tok % U) / TT, tok, i, kg);
    };
    // bit x: this lane's V block of the sub-tile staged in slot x is a real
    // block (recorded when its loads are issued, read by the math)
    uint32_t okbits = 0;
    // Stage sub-tile s in LDS slot `slot` with global-to-LDS loads: the
    // workgroup's 256 threads move its KG + VG 16-byte groups, group
    // x = 256u + 64 * wave + lane being load x / 64 of lane x % 64 (K loads
    // first, then V), so that a wavefront later reads group m * 64 + lane as
    // its m-th load.  Each load writes 16 bytes per lane at the wavefront's
    // LDS base + 16 * lane.
    constexpr int NG = (KG + VG) / 256;
    const uint32_t lds0 = uniform((uint32_t)(uintptr_t)lds);
    auto issue = [&](int32_t s, int slot) {
      const Addr a = where(s);
      okbits = a.ok ? okbits | (1u << slot) : okbits & ~(1u << slot);
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int x0 = 256 * u + 64 * wv;  // uniform
        const uint8_t* src;
        if (x0 < KG) {
          const int m = x0 >> 6;            // QK tile m / NKJ, step m % NKJ
          src = a.krow + (4 * (m % NKJ) * BS + 4 * (m / NKJ)) * 16;
        } else {
          src = a.vrow + 16 * ((x0 - KG) >> 6) * VT * EB;
        }
        lds_dma16(src, lds0 + (uint32_t)(slot * STAGE_BYTES + x0 * 16));
      }
    };

    // Sub-tiles below s_full need no masking in this wavefront: every live
    // row attends all of their tokens (rows that are not live produce
    // nothing, whatever they compute), and all their blocks are real.
    int32_t lmin = INT32_MAX;
#pragma unroll
    for (int t = 0; t < NT; ++t) lmin = min(lmin, live[t] ? Lc[t] : INT32_MAX);
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) lmin = min(lmin, __shfl_xor(lmin, x));
    int32_t s_full = uniform(lmin / TT);
    {
      // the first table entry of the chunk that is not a real block
      const int32_t e0 = (int32_t)((int64_t)s0 * TT / BS);
      const int32_t e1 = min(P.shared, (int32_t)(((int64_t)s1 * TT + BS - 1) / BS));
      for (int32_t e = e0; e < e1; e += 64) {
        const int32_t k = e + lane;
        const int32_t id = k < e1 ? P.tables[k] : 0;
        const uint64_t bad = __ballot(k < e1 && (id < 0 || id >= P.num_blocks));
        if (bad) {
          s_full = min(s_full, (int32_t)((int64_t)(e + __builtin_ctzll(bad)) * BS / TT));
          break;
        }
      }
    }

    const float scale_abs = __builtin_fabsf(P.scale_log2);
    if (s0 < s1) {
      // STAGES LDS slots: STAGES - 1 sub-tiles in flight while one is used;
      // sub-tile x lives in slot (x - s0) % STAGES
      for (int k = 0; k < STAGES - 1 && s0 + k < s1; ++k) issue(s0 + k, k);
      int slot = 0;
      // Sub-tile s into K and V.  It has landed once no more than `ahead`
      // stages (NG loads each) are outstanding: this thread's, then (barrier)
      // every thread's.  After the barrier every wavefront is also done with
      // the slot of sub-tile s - 1, which the next issue refills.
      auto next = [&](int32_t s, KTile& K, VTile& V) {
        const int ahead = min(STAGES - 2, s1 - 1 - s);
        wait_stages<NG, STAGES - 2>(ahead);
        __syncthreads();
        if (s + STAGES - 1 < s1) issue(s + STAGES - 1, slot == 0 ? STAGES - 1 : slot - 1);
        const uint4* src = reinterpret_cast<const uint4*>(lds + slot * STAGE_BYTES);
#pragma unroll
        for (int m = 0; m < NKL; ++m) K.k[m] = src[m * 64 + lane];
#pragma unroll
        for (int n = 0; n < NV; ++n) V.v[n] = src[KG + n * 64 + lane];
        V.tok0 = s * TT;
        V.ok = ((okbits >> slot) & 1u) != 0;
        slot = slot == STAGES - 1 ? 0 : slot + 1;
      };
      // the sub-tiles that need no masking, then the rest
      const int32_t s_mid = max(s0, min(s1, s_full));
      for (int32_t s = s0; s < s_mid; ++s) {
        KTile K;
        VTile V;
        next(s, K, V);
        prefix_step<false>(K, V, q, st, Lc, kT, scale_abs, kg);
      }
      for (int32_t s = s_mid; s < s1; ++s) {
        KTile K;
        VTile V;
        next(s, K, V);
        prefix_step<true>(K, V, q, st, Lc, kT, scale_abs, kg);
      }
    }

    float vsc[NV][4];
    v_scales(P, g, kg, vsc);
    const int64_t bhq = (int64_t)P.batch * P.hq;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float l1 = st[t].l + __shfl_xor(st[t].l, 16);
      const float lall = l1 + __shfl_xor(l1, 32);
      if (!live[t]) continue;
      float* base = P.ws_pre + ((int64_t)c * bhq + hrow[t]) * PRE_STRIDE;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = st[t].O[n][r] * vsc[n][r];
        *reinterpret_cast<f32x4*>(base + 16 * n + 4 * kg) = o;
      }
      if (kg == 0) *reinterpret_cast<f32x2*>(base + D) = f32x2{st[t].m, lall};
    }
  }

  // One wavefront's units [r0, r1) (KV-head-major global unit indices; the
  // first lies in pair (g0, b0)) as one stream of sub-tiles: the loads run
  // one sub-tile ahead of the math across piece boundaries, and the next
  // piece's queries (FP8: also its first block-table entries) are fetched
  // while the current piece streams.  C: unit prefix sums (NULL in single
  // mode, where the range is the whole of one pair).
  static __device__ void stream(const DecodeParams& P, const int32_t* C, int64_t t_head, int64_t T, int64_t W,
                                int64_t w, int64_t r0, int64_t r1, int g0, int b0, uint8_t* stage) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int kg = lane >> 4;

    // load side: the piece whose sub-tiles are being fetched
    Seg ls = make_seg(P, C, t_head, g0, b0);
    if (!C) r1 = r0 + ls.nb;
    int64_t lbeg = r0;
    int64_t lend = min(r1, ls.start + ls.nb);
    int32_t tb0, tb1;
    piece_blocks(ls, lbeg, lend, &tb0, &tb1);
    // Block-table entries: FP8 reads them 64 at a time, one per lane (the
    // next 64 and the next piece's first 64 prefetched); the other types read
    // each sub-tile's entries with scalar loads.  A vector load of entries
    // for a later sub-tile needs a register copy where the code paths join,
    // and the copy waits for every load in flight; scalar loads are counted
    // apart from the vector loads.
    constexpr bool SCALAR_TABLE = KV != KV_FP8;
    int32_t tcur = -1, tnext = -1;
    if constexpr (!SCALAR_TABLE) {
      tcur = table_chunk(P, ls.b, tb0, tb1, 0, lane);
      tnext = tb1 - tb0 > 64 ? table_chunk(P, ls.b, tb0, tb1, 1, lane) : -1;
    }
    int ccur = 0;
    // the piece after it, with its first table entries in flight (looked up
    // once the first sub-tile's loads are out)
    Seg ln = ls;
    bool has_ln = false;
    int32_t tpn = -1;
    qop q[NQ], qn[NQ];
    load_q(P, ls.b, ls.g, i, kg, q);

    // compute side: the piece whose sub-tiles are being scored
    Seg cs = ls;
    int64_t cbeg = lbeg, cend = lend;

    int64_t lx = r0;  // unit and sub-tile of the next load
    int lsub = 0;
    auto where = [&](bool& last) -> Addr {
      if (lx == lend) {
        // enter the next piece
        ls = ln;
        lbeg = lend;
        lend = min(r1, ls.start + ls.nb);
        piece_blocks(ls, lbeg, lend, &tb0, &tb1);
        if constexpr (!SCALAR_TABLE) {
          tcur = tpn;
          tnext = tb1 - tb0 > 64 ? table_chunk(P, ls.b, tb0, tb1, 1, lane) : -1;
          ccur = 0;
        }
        load_q(P, ls.b, ls.g, i, kg, qn);
        has_ln = lend < r1 && next_seg(P, C, t_head, ls, ln);
        if constexpr (!SCALAR_TABLE) {
          if (has_ln) {
            int32_t nb0, nb1;
            piece_blocks(ln, ln.start, min(r1, ln.start + ln.nb), &nb0, &nb1);
            tpn = table_chunk(P, ln.b, nb0, nb1, 0, lane);
          }
        }
      }
      const int rel = (int)(lx - lbeg) * UB;
      int32_t ids[UB];
      if constexpr (SCALAR_TABLE) {
        table_entries_scalar<UB>(P.tables + (int64_t)ls.b * P.max_blocks + tb0, rel, tb1 - tb0, ids);
      } else {
        const int c = rel >> 6;
        if (c != ccur) {
          tcur = tnext;
          tnext = tb0 + 64 * (c + 1) < tb1 ? table_chunk(P, ls.b, tb0, tb1, c + 1, lane) : -1;
          ccur = c;
        }
#pragma unroll
        for (int k = 0; k < UB; ++k) ids[k] = __builtin_amdgcn_readlane(tcur, (rel & 63) + k);
      }
      const Addr a = locate(P, ls.g, ids, lsub, (tb0 + rel) * BS + lsub * TT, i, kg);
      last = lsub == SPU - 1 && lx + 1 == lend;
      if (++lsub == SPU) {
        lsub = 0;
        ++lx;
      }
      return a;
    };

    State st;
    auto reset = [&]() {
#pragma unroll
      for (int n = 0; n < NV; ++n) st.O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.m = -INFINITY;
      st.l = 0.f;
    };
    reset();
    // after the last sub-tile of a piece: write it, then take over the piece
    // the loads have moved on to.  While the range goes on, the piece's
    // result is kept in LDS when there is room: a store issued now would sit
    // in the same in-order wait counter as the loads in flight, and the next
    // waits for sub-tiles would also wait for its acknowledgement.
    int nst = 0;
    auto step_piece = [&](bool more) {
      if (more && nst < P.nstage) stage_put(stage, P.nstage, nst++, P.group, st, cs, cbeg, cend, i, kg, lane);
      else finish(P, st, cs, cbeg, cend, r0, T, W, w, i, kg, lane);
      if (more) {
        cs = ls;
        cbeg = lbeg;
        cend = lend;
#pragma unroll
        for (int k = 0; k < NQ; ++k) q[k] = qn[k];
        reset();
      }
    };

    // Pipeline over sub-tiles in two register buffers: the K and V loads of
    // sub-tile s+1 are in flight while s is scored and accumulated.
    const int64_t nsub = (r1 - r0) * SPU;
    KTile K0, K1;
    VTile V0, V1;
    f32x4 S[NQT];
    float p[NQT][4];
    bool last0, last1;
    Addr a0 = where(last0);
    Addr a1 = a0;
    load_k(K0, a0);
    load_v(V0, a0);
    __builtin_amdgcn_sched_barrier(0);
    has_ln = C && lend < r1 && next_seg(P, C, t_head, ls, ln);
    if constexpr (!SCALAR_TABLE) {
      if (has_ln) {
        int32_t nb0, nb1;
        piece_blocks(ln, ln.start, min(r1, ln.start + ln.nb), &nb0, &nb1);
        tpn = table_chunk(P, ln.b, nb0, nb1, 0, lane);
      }
    }
    // sched_barrier keeps the compiler from hoisting the next sub-tile's
    // loads above the current one's math (that would hold three half-tiles
    // at once and spill).
    for (int64_t s = 0; s < nsub; s += 2) {
      const bool n1 = s + 1 < nsub;
      if (n1) {
        a1 = where(last1);
        load_k(K1, a1);
        load_v(V1, a1);
      }
      __builtin_amdgcn_sched_barrier(0);
      qk(K0, q, S);
      softmax(V0, S, st, p, cs.lo, cs.L, P.scale_log2, kg);
      __builtin_amdgcn_sched_barrier(0);
      pv(V0, p, st, cs.lo, cs.L, kg);
      __builtin_amdgcn_sched_barrier(0);
      if (last0) step_piece(n1);
      if (!n1) break;
      const bool n2 = s + 2 < nsub;
      if (n2) {
        a0 = where(last0);
        load_k(K0, a0);
        load_v(V0, a0);
      }
      __builtin_amdgcn_sched_barrier(0);
      qk(K1, q, S);
      softmax(V1, S, st, p, cs.lo, cs.L, P.scale_log2, kg);
      __builtin_amdgcn_sched_barrier(0);
      pv(V1, p, st, cs.lo, cs.L, kg);
      __builtin_amdgcn_sched_barrier(0);
      if (last1) step_piece(n2);
    }
    // the staged pieces, now that no load is in flight (their tags were
    // written by lane 0 and are read by every lane: keep the reads below)
    asm volatile("" ::: "memory");
    for (int k = 0; k < nst; ++k) {
      Seg ps;
      int64_t pbeg, pend;
      stage_get(stage, P.nstage, k, P.group, st, ps, &pbeg, &pend, i, kg);
      finish(P, st, ps, pbeg, pend, r0, T, W, w, i, kg, lane);
    }
  }
};

// Fused append, workgroup a of an append part: the new tokens of sequences
// a * spg .. a * spg + spg - 1 (spg = P.append_spg) into the pool (every KV
// head).  A slot outside the pool is not written.  The slots are read first,
// one load per sequence; every thread then loads its token chunk whole and
// stores it.
//  - ROWS = false: workgroups after decode_kernel's own, so that they run in
//    its tail.  Each row's slot goes to ws_slots, and merge_kernel writes the
//    rows' table entries and lengths, which the decode reads.  The token's
//    slot is a position of its own row past the cached tokens (a block
//    block_table_append made the row's own by copy-on-write), which no
//    wavefront attends as a cached token.
//  - ROWS = true: the first workgroups of merge_kernel (FP8 pools), after
//    the decode; they also write each row's table entry and length.
template <int D, int KV, int SRC, bool ROWS>
__device__ void append_group(const DecodeParams& P, const TailParams& T, int a) {
  __shared__ int64_t sl[16];
  const int tid = threadIdx.x;
  const int b0 = a * P.append_spg;
  const int nb = min(P.append_spg, P.batch - b0);
  const int64_t cap = P.num_blocks * P.block_size;
  if (tid < nb) {
    const int b = b0 + tid;
    const int64_t slot = __hip_atomic_load(P.new_slots + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    sl[tid] = slot;
    if constexpr (ROWS) {
      if (slot >= 0 && slot < cap) {
        const int32_t L = P.lens_w[b];
        if (L >= 0 && L / P.block_size < P.max_blocks) {
          // the row's table entry for the token's block and its new length
          P.tables_w[(int64_t)b * P.max_blocks + L / P.block_size] = (int32_t)(slot / P.block_size);
          P.lens_w[b] = L + 1;
        }
      }
    } else {
      T.ws_slots[b] = slot;
    }
  }
  __syncthreads();
  constexpr int chunks = D / (16 / Elem<KV>::bytes);
  const int per = P.hkv * chunks;
  uint8_t* kc = const_cast<uint8_t*>(P.kc);
  uint8_t* vc = const_cast<uint8_t*>(P.vc);
  for (int t = tid; t < nb * per; t += blockDim.x) {
    const int i = t / per;
    const int64_t slot = sl[i];
    if (slot < 0 || slot >= cap) continue;
    const int h = (t / chunks) % P.hkv;
    const TokenChunk<KV, SRC> tok = load_token_chunk<KV, SRC>(P.new_k, P.new_v, P.k_inv, P.v_inv, P.hkv, D,
                                                              P.layer, ((int64_t)(b0 + i) * P.hkv + h) * D,
                                                              t % chunks, h);
    store_token_chunk<KV, SRC>(tok, kc, vc, P.num_blocks, P.hkv, D, P.block_size, P.layer, t % chunks, h,
                               slot / P.block_size, (int)(slot % P.block_size));
  }
}

// Workgroups at the front of the fused merge: the FP8 append groups, or
// one per 256 rows for the rows' tables and lengths.
__host__ __device__ inline int64_t merge_row_groups(const DecodeParams& P) {
  return P.kv_dtype == PKV_FP8_E4M3 ? (P.batch + P.append_spg - 1) / P.append_spg : (P.batch + 255) / 256;
}

// Fused append, after the decode: rows a * 256 .. a * 256 + 255 take the
// token's block as their table entry at L / block_size and L + 1 as their
// length (a slot outside the pool, or no room in the table: neither).
__device__ void update_rows(const DecodeParams& P, const TailParams& T, int a) {
  const int b = a * 256 + (int)threadIdx.x;
  if (b >= P.batch) return;
  const int64_t slot = T.ws_slots[b];
  const int32_t L = P.lens_w[b];
  const int64_t cap = P.num_blocks * P.block_size;
  if (slot >= 0 && slot < cap && L >= 0 && L / P.block_size < P.max_blocks) {
    P.tables_w[(int64_t)b * P.max_blocks + L / P.block_size] = (int32_t)(slot / P.block_size);
    P.lens_w[b] = L + 1;
  }
}

template <int KV, int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_kernel(DecodeParams P) {
  typedef Decoder<KV, D, BS> Dec;
  constexpr int U = Units<KV, BS>::U;
  extern __shared__ int32_t C[];
  const int lane = threadIdx.x & 63;
  const int wid = uniform((int)(threadIdx.x >> 6));  // wave-uniform: keeps all work indices scalar
  int64_t wg = blockIdx.x;
  if (P.xcd_remap) wg = (wg % 8) * (gridDim.x / 8) + wg / 8;
  const int64_t w = wg * 4 + wid;

  if (P.single) {
    // one wavefront per (KV head, sequence), KV-head major
    if (w >= (int64_t)P.hkv * P.batch) return;
    const int g = (int)(w / P.batch);
    const int b = (int)(w % P.batch);
    int32_t L, lo, first, nu;
    seq_extent<BS, U>(P, b, &L, &lo, &first, &nu);
    if (nu == 0) {
      // nothing cached to attend: zeros, or (fused append) the new token
      // alone, which merge_kernel writes
      if (!P.allpart) write_zero_rows<D>(P, b, g, lane);
      else if (lane == 0) P.ws_job[w] = make_int4(0, 0, 0, 0);
      return;
    }
    Dec::stream(P, nullptr, 0, 0, 0, 0, 0, 0, g, b, nullptr);
    return;
  }

  scan_units<BS, U>(P, C);
  const int64_t t_head = C[P.batch];
  const int64_t T = t_head * P.hkv;
  // sequences with nothing to attend get zero rows
  const int64_t nseg = (int64_t)P.hkv * P.batch;
  const int64_t launched = (int64_t)gridDim.x * 4;
  for (int64_t seg = w; seg < nseg; seg += launched) {
    const int b = (int)(seg % P.batch);
    if (C[b + 1] == C[b]) {
      // nothing of its own to attend: zeros, or (shared prefix, fused append)
      // the merge of the prefix partials and the new token alone, written by
      // merge_kernel
      if (!P.allpart) write_zero_rows<D>(P, b, (int)(seg / P.batch), lane);
      if (lane == 0) P.ws_job[seg] = make_int4(0, 0, 0, 0);
    }
  }
  if (w >= P.num_waves) return;
  // all units of all (KV head, sequence) pairs laid end to end, KV-head
  // major, cut into W equal non-empty ranges
  const int64_t W = P.num_waves < T ? P.num_waves : T;
  if (w < W) {
    const int64_t r0 = range_start(w, T, W);
    const int64_t r1 = range_start(w + 1, T, W);
    const int g = (int)(r0 / t_head);
    const int32_t r = (int32_t)(r0 % t_head);
    // largest b with C[b] <= r: the pair holding unit r0 (it has units)
    int lo_b = 0, hi_b = P.batch - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (C[mid] <= r) lo_b = mid;
      else hi_b = mid - 1;
    }
    uint8_t* stage = reinterpret_cast<uint8_t*>(C) + P.stage_off + wid * Dec::stage_area_bytes(P.group, P.nstage);
    Dec::stream(P, C, t_head, T, W, w, r0, r1, g, uniform(lo_b), stage);
  }
}

// decode_kernel's body for decode_append_kernel: the decode over the first
// nwg workgroups of the grid.  The same steps as decode_kernel (which uses
// the whole grid); decode_kernel keeps its own copy because its generated
// code, the FP8 one above all, changed and slowed when it was built from a
// shared body.
template <int KV, int D, int BS>
__device__ __forceinline__ void decode_body(DecodeParams P, uint32_t nwg) {
  typedef Decoder<KV, D, BS> Dec;
  constexpr int U = Units<KV, BS>::U;
  extern __shared__ int32_t C[];
  const int lane = threadIdx.x & 63;
  const int wid = uniform((int)(threadIdx.x >> 6));  // wave-uniform: keeps all work indices scalar
  int64_t wg = blockIdx.x;
  if (P.xcd_remap) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int64_t w = wg * 4 + wid;

  if (P.single) {
    // one wavefront per (KV head, sequence), KV-head major
    if (w >= (int64_t)P.hkv * P.batch) return;
    const int g = (int)(w / P.batch);
    const int b = (int)(w % P.batch);
    int32_t L, lo, first, nu;
    seq_extent<BS, U>(P, b, &L, &lo, &first, &nu);
    if (nu == 0) {
      // nothing cached to attend: zeros, or (fused append) the new token
      // alone, which merge_kernel writes
      if (!P.allpart) write_zero_rows<D>(P, b, g, lane);
      else if (lane == 0) P.ws_job[w] = make_int4(0, 0, 0, 0);
      return;
    }
    Dec::stream(P, nullptr, 0, 0, 0, 0, 0, 0, g, b, nullptr);
    return;
  }

  scan_units_wave<BS, U>(P, C);
  const int64_t t_head = C[P.batch];
  const int64_t T = t_head * P.hkv;
  // sequences with nothing to attend get zero rows
  const int64_t nseg = (int64_t)P.hkv * P.batch;
  const int64_t launched = (int64_t)nwg * 4;
  for (int64_t seg = w; seg < nseg; seg += launched) {
    const int b = (int)(seg % P.batch);
    if (C[b + 1] == C[b]) {
      // nothing of its own to attend: zeros, or (shared prefix, fused append)
      // the merge of the prefix partials and the new token alone, written by
      // merge_kernel
      if (!P.allpart) write_zero_rows<D>(P, b, (int)(seg / P.batch), lane);
      if (lane == 0) P.ws_job[seg] = make_int4(0, 0, 0, 0);
    }
  }
  if (w >= P.num_waves) return;
  // all units of all (KV head, sequence) pairs laid end to end, KV-head
  // major, cut into W equal non-empty ranges
  const int64_t W = P.num_waves < T ? P.num_waves : T;
  if (w < W) {
    const int64_t r0 = range_start(w, T, W);
    const int64_t r1 = range_start(w + 1, T, W);
    const int g = (int)(r0 / t_head);
    const int32_t r = (int32_t)(r0 % t_head);
    // largest b with C[b] <= r: the pair holding unit r0 (it has units)
    int lo_b = 0, hi_b = P.batch - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (C[mid] <= r) lo_b = mid;
      else hi_b = mid - 1;
    }
    uint8_t* stage = reinterpret_cast<uint8_t*>(C) + P.stage_off + wid * Dec::stage_area_bytes(P.group, P.nstage);
    Dec::stream(P, C, t_head, T, W, w, r0, r1, g, uniform(lo_b), stage);
  }
}

// The decode of a call with a fused append (pools other than FP8): the
// workgroups past the decode's store the new tokens in its tail.  A kernel
// of its own so that the plain decode's code is not changed by it (the FP8
// decode, whose scalar registers are at their limit, slowed when it held
// this path).
template <int KV, int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_append_kernel(
    DecodeParams P, TailParams TP) {
  if ((int)blockIdx.x >= TP.decode_wgs) {
    append_group<D, KV, KV, false>(P, TP, (int)blockIdx.x - TP.decode_wgs);
    return;
  }
  decode_body<KV, D, BS>(P, (uint32_t)TP.decode_wgs);
}

// Shared prefix: workgroup x takes (KV head g, row group rg, token chunk c),
// KV-head major, so the workgroups of one head sit on one XCD and its prefix
// blocks stay in that XCD's L2.
template <int KV, int D, int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefix_kernel(DecodeParams P) {
  typedef Decoder<KV, D, BS> Dec;
  __shared__ __attribute__((aligned(16))) uint8_t stage[Dec::STAGES * Dec::STAGE_BYTES];
  int64_t wg = blockIdx.x;
  wg = (wg % 8) * (gridDim.x / 8) + wg / 8;
  const int64_t per_head = (int64_t)P.pre_rtiles * P.pre_chunks;
  if (wg >= per_head * P.hkv) return;   // whole workgroup: no barrier is skipped
  const int g = (int)(wg / per_head);
  const int64_t rem = wg % per_head;
  Dec::prefix_group(P, g, (int)(rem / P.pre_chunks), (int)(rem % P.pre_chunks), stage);
}

// The value the pool holds for a source value x of one channel: x itself,
// or (FP8) the E4M3 code of x * inv decoded and times the channel's scale --
// what the decode reads back.
template <int KV>
__device__ __forceinline__ float pool_value(float x, float inv, float scale) {
  if constexpr (KV != KV_FP8) {
    return x;
  } else {
    const uint32_t code = f32_to_e4m3(x * inv);
    const bf16x2 w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false);
    return (float)w[0] * scale;
  }
}

// Sequences whose new tokens one append workgroup of merge_kernel writes: as
// many as give its 256 threads one token chunk (16 bytes of K and its V
// elements) each -- every thread's loads then go out in one round trip --
// and at most 16, whose slots are read with one coalesced load.
static int append_seqs_per_group(int hkv, int d, int kv_dtype) {
  const int chunks = d / (kv_dtype == PKV_F32 ? 4 : (kv_dtype == PKV_FP8_E4M3 ? 16 : 8));
  return std::max(1, std::min(16, 256 / (hkv * chunks)));
}

// Elements lane, lane + 64, ... of a row of D (element type T), as fp32.
template <int D, int T>
__device__ __forceinline__ void load_row(const uint8_t* p, int64_t row, int lane, float (&v)[D / 64]) {
#pragma unroll
  for (int e = 0; e < D / 64; ++e) v[e] = src_to_f32<T>(p, row + lane + 64 * e);
}

// Log-sum-exp merge of the pieces of a split (KV head, sequence).  Merge
// workgroup x < segs * pg is (seg, y) = (x / pg, x % pg) (with pg = 1, x
// first spread over the XCDs, below); it owns a contiguous share of the
// G * D/4 output positions (head h, 4 dims) of sequence-head seg; TPP
// threads share a position, thread sub taking pieces sub, sub + TPP, ...
// Each thread loads the (max, sum) and o of up to NPC of its pieces at once,
// so the partials are read in one round trip after the job; more pieces are
// folded in batches of NPC with the usual rescaling.  The thread maxima are
// combined by lane exchanges, then the rescaled sums by a butterfly that
// leaves the same bits in every lane of a position (deterministic).  Piece p
// of a job whose first piece is in range w0 is in slot (w0, first) for p = 0
// and (w0 + p, 0) after.
//
// With a fused append (NKV >= 0: pool dtype NKV, source dtype NSRC) the new
// token is one more partial of every (sequence, head): o = its V row, max =
// its score, sum = 1.  Its K elements, channel scales and the query rows
// are loaded with the job, its V elements before the partials; its scores
// (one wavefront per head, lanes over the dims) are computed after the
// partials' loads have gone out, and the first thread of each position
// folds it in.  The dtypes are compile-time constants so that these loads
// are straight-line code and go out together.  The first workgroups of this
// grid write the rows' table entries and lengths (update_rows; the tokens
// are already in the pool, stored in the decode's tail), or for an FP8 pool
// store the tokens too (append_group).  Kept out of the FP8 decode, that
// code slowed its stream loop.
template <int D, int NKV, int NSRC>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams P, TailParams TP) {
  constexpr int NPC = 4;   // pieces per thread per batch
  constexpr bool FUSED = NKV >= 0;
  constexpr int KV = FUSED ? NKV : KV_F32;
  constexpr int SRC = FUSED ? NSRC : KV_F32;
  constexpr int QT = KV == KV_FP8 ? KV_BF16 : KV;   // the queries' dtype
  // fused append: the first workgroups write the rows' table entries and
  // lengths (the decode, which reads them, has finished), and for an FP8
  // pool also store the new tokens
  int64_t nmeta = 0;
  if constexpr (FUSED) {
    // their count padded to a multiple of 8, so that the merge workgroups
    // after them start on XCD 0
    const int64_t nreal = merge_row_groups(P);
    nmeta = (nreal + 7) / 8 * 8;
    if ((int64_t)blockIdx.x < nmeta) {
      if ((int64_t)blockIdx.x < nreal) {
        if constexpr (KV == KV_FP8) append_group<D, KV, SRC, true>(P, TP, (int)blockIdx.x);
        else update_rows(P, TP, (int)blockIdx.x);
      }
      return;
    }
  }
  // With one workgroup per sequence-head and a multiple of 8 of them, the
  // workgroups on one XCD take a contiguous eighth of the sequence-heads
  // (KV-head major), the ones whose pieces the decode's wavefront ranges on
  // that XCD wrote: the partials are read back on the XCD that wrote them.
  int64_t x = blockIdx.x - nmeta;
  {
    const int64_t segs = (int64_t)P.batch * P.hkv;
    if (P.merge_pg == 1 && segs % 8 == 0) x = (x % 8) * (segs / 8) + x / 8;
  }
  const int64_t seg = x / P.merge_pg;
  const int yb = (int)(x % P.merge_pg);
  const int b = (int)(seg % P.batch), g = (int)(seg / P.batch);
  const int G = P.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int4 job = P.ws_job[seg];
  __shared__ float s_new[16];          // log2-domain score of the new token, per head of the group
  const int64_t s0 = ((int64_t)P.layer * P.hkv + g) * D;   // channel scales of (layer, KV head)
  // fused append: the new token's K elements lane, lane + 64, ... (with their
  // channel scales) and the query rows of heads wv, wv + 4, ... of the group
  // (at most 4 per wavefront: G <= 16)
  float kx[D / 64], ki[D / 64], ks[D / 64], q[4][D / 64];
  if constexpr (FUSED) {
    load_row<D, SRC>(P.new_k, ((int64_t)b * P.hkv + g) * D, lane, kx);
    if constexpr (KV == KV_FP8) {
#pragma unroll
      for (int e = 0; e < D / 64; ++e) {
        ki[e] = P.k_inv[s0 + lane + 64 * e];
        ks[e] = P.k_scale[s0 + lane + 64 * e];
      }
    }
    // rows past the group repeat its last head (never used): no branch
    // around a load, so that every load goes out before the first wait
#pragma unroll
    for (int u = 0; u < 4; ++u)
      load_row<D, QT>(P.q, ((int64_t)b * P.hq + (int64_t)g * G + min(wv + 4 * u, G - 1)) * D, lane, q[u]);
  }
  const int npieces = job.y;
  if (!FUSED && npieces == 0 && !P.allpart) return;
  const int64_t w0 = job.x;
  const int first_which = job.z;
  constexpr int D4 = D / 4;
  const int NP = G * D4;
  const int npg = (NP + P.merge_pg - 1) / P.merge_pg;
  const int pos0 = yb * npg;
  const int pos1 = min(NP, pos0 + npg);
  int tpp = 1;
  while (tpp * 2 * npg <= 256 && tpp < 64) tpp *= 2;   // threads per position (lanes of one wavefront)
  const int sub = tid % tpp;
  // a trip count uniform over the workgroup (a fused append has a barrier in
  // the first trip); threads past pos1 only take part in it
  const int per_trip = 256 / tpp;
  const int trips = (pos1 - pos0 + per_trip - 1) / per_trip;
  for (int trip = 0; trip < trips; ++trip) {
    const int pos_raw = pos0 + tid / tpp + trip * per_trip;
    const bool active = pos_raw < pos1;
    const int pos = active ? pos_raw : pos0;
    const int h = pos / D4;
    const int d4 = (pos % D4) * 4;
    // the new token's V elements of this position (and their channel
    // scales), loaded before the partials and converted after them
    f32x4 vraw = {0.f, 0.f, 0.f, 0.f};
    uint2 vbits = {0u, 0u};
    float vi[4], vs[4];
    if constexpr (FUSED) {
      if (sub == 0) {
        const int64_t e0 = ((int64_t)b * P.hkv + g) * D + d4;    // 4 consecutive elements, one load
        if constexpr (SRC == KV_F32)
          vraw = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(P.new_v) + e0);
        else
          vbits = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(P.new_v) + e0);
        if constexpr (KV == KV_FP8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vi[e] = P.v_inv[s0 + d4 + e];
            vs[e] = P.v_scale[s0 + d4 + e];
          }
        }
      }
    }
    auto slot_of = [&](int pc) -> int64_t { return ((w0 + pc) * 2 + (pc == 0 ? first_which : 0)) * G + h; };
    float M = -INFINITY, Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = sub; base < npieces; base += NPC * tpp) {
      f32x2 ml[NPC];
      f32x4 o[NPC];
#pragma unroll
      for (int k = 0; k < NPC; ++k) {
        const int pc = base + k * tpp;
        if (pc < npieces) {
          const int64_t sl = slot_of(pc);
          ml[k] = *reinterpret_cast<const f32x2*>(P.ws_ml + sl * 2);
          o[k] = *reinterpret_cast<const f32x4*>(P.ws_o + sl * D + d4);
        } else {
          ml[k] = f32x2{-INFINITY, 0.f};
          o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < NPC; ++k) Mb = fmaxf(Mb, ml[k][0]);
      const float Mu = Mb == -INFINITY ? 0.f : Mb;
      const float r = __builtin_amdgcn_exp2f(M - Mu);
      acc *= r;
      Ls *= r;
#pragma unroll
      for (int k = 0; k < NPC; ++k) {
        const float wt = __builtin_amdgcn_exp2f(ml[k][0] - Mu);
        acc += o[k] * wt;
        Ls += ml[k][1] * wt;
      }
      M = Mb;
    }
    // the prefix partials of this (sequence, head), and (job.w) the partial
    // of its own part when one wavefront held all of it: same fold, also up
    // to NPC partials per thread per round trip
    if (P.allpart) {
      const int64_t bhq = (int64_t)P.batch * P.hq;
      const int64_t hrow = (int64_t)b * P.hq + (int64_t)g * G + h;
      const int nslots = P.pre_chunks + (job.w ? 1 : 0);
      for (int cb = sub; cb < nslots; cb += NPC * tpp) {
        f32x2 ml[NPC];
        f32x4 o[NPC];
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
          const int cc = cb + k * tpp;
          if (cc < nslots) {
            const float* base = P.ws_pre + ((int64_t)cc * bhq + hrow) * (D + 4);
            ml[k] = *reinterpret_cast<const f32x2*>(base + D);
            o[k] = *reinterpret_cast<const f32x4*>(base + d4);
          } else {
            ml[k] = f32x2{-INFINITY, 0.f};
            o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < NPC; ++k) Mb = fmaxf(Mb, ml[k][0]);
        const float Mu = Mb == -INFINITY ? 0.f : Mb;
        const float r = __builtin_amdgcn_exp2f(M - Mu);
        acc *= r;
        Ls *= r;
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
          const float wt = __builtin_amdgcn_exp2f(ml[k][0] - Mu);
          acc += o[k] * wt;
          Ls += ml[k][1] * wt;
        }
        M = Mb;
      }
    }
    // the new token: one more partial (its V row, its score, sum 1), folded
    // in by one thread of the position
    if constexpr (FUSED) {
      if (trip == 0) {
        // its scores, heads wv, wv + 4, ... on wavefront wv: the four sums
        // are reduced together, so that their lane exchanges overlap
        float kv[D / 64];
#pragma unroll
        for (int e = 0; e < D / 64; ++e) kv[e] = pool_value<KV>(kx[e], ki[e], ks[e]);
        float dot[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          dot[u] = 0.f;
#pragma unroll
          for (int e = 0; e < D / 64; ++e) dot[u] += q[u][e] * kv[e];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
          for (int u = 0; u < 4; ++u) dot[u] += __shfl_xor(dot[u], off);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (lane == 0 && wv + 4 * u < G) s_new[wv + 4 * u] = dot[u] * P.scale_log2;
        __syncthreads();
      }
      if (sub == 0) {
        f32x4 vn;
        if constexpr (SRC == KV_F32) {
          vn = vraw;
        } else {
          const uint32_t h16[4] = {vbits.x & 0xffffu, vbits.x >> 16, vbits.y & 0xffffu, vbits.y >> 16};
#pragma unroll
          for (int e = 0; e < 4; ++e) vn[e] = SRC == KV_F16 ? f16_bits_to_f32(h16[e]) : bf16_bits_to_f32(h16[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) vn[e] = pool_value<KV>(vn[e], vi[e], vs[e]);
        const float sn = s_new[h];
        const float Mb = fmaxf(M, sn);
        const float r = __builtin_amdgcn_exp2f(M - Mb);     // M = -inf: 0
        const float wt = __builtin_amdgcn_exp2f(sn - Mb);
        acc = acc * r + vn * wt;
        Ls = Ls * r + wt;
        M = Mb;
      }
    }
    // combine the tpp threads of the position: common max, rescale, sum
    float Mall = M;
    for (int off = 1; off < tpp; off <<= 1) Mall = fmaxf(Mall, __shfl_xor(Mall, off));
    const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mall);
    acc *= r;
    Ls *= r;
    for (int off = 1; off < tpp; off <<= 1) {
      Ls += __shfl_xor(Ls, off);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
    }
    if (sub == 0 && active) {
      const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
      store4(P, ((int64_t)b * P.hq + (int64_t)g * G + h) * D + d4, acc * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// HBM read probe (measurement only): the buffer read once with the 16-byte
// streaming loads the decode uses for K and V.  Workgroup x reads one
// contiguous chunk, four loads in flight per thread per round; the XOR of
// what a thread read is stored only if it equals `tag`, so that the loads
// cannot be dropped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ sink, uint32_t tag) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  int64_t x = beg + threadIdx.x;
  for (; x + 3 * 256 < end; x += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + x + u * 256);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; x < end; x += 256) {
    const u32x4 v = __builtin_nontemporal_load(p + x);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == tag) sink[0] = acc;
}

// ---------------------------------------------------------------------------
// metadata upload: page-locked host memory -> device memory, by a kernel
// ---------------------------------------------------------------------------
// A copy engine would need a hand-off between two hardware queues before and
// after the copy; a kernel on the caller's stream is ordered like the kernels
// around it.  The loads are system-scope atomics, so they see what the host
// wrote before the launch whatever the GPU caches hold.
__global__ __launch_bounds__(256) void upload_kernel(const uint64_t* __restrict__ src,
                                                     uint64_t* __restrict__ dst, int64_t n8,
                                                     const uint32_t* __restrict__ src_tail,
                                                     uint32_t* __restrict__ dst_tail) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __hip_atomic_load(src + i + u * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n8; i += stride)
    dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (src_tail && blockIdx.x == 0 && threadIdx.x == 0)
    *dst_tail = __hip_atomic_load(src_tail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static constexpr int kWavesPerCU = 4;
static constexpr int64_t kMaxWaves = 16384;   // largest split count
static constexpr int kMaxBatch = 16000;   // C[] of B+1 ints in LDS

static pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static constexpr int kMaxDevices = 64;

static pkv_status device_cus(int* cus) {
  static std::mutex mu;
  static int cache[kMaxDevices];   // fixed size: no host allocation on a launch path
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_E_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(mu);
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
  if (a->num_splits > kMaxWaves) return fail(PKV_E_UNSUPPORTED, "num_splits above 16384");
  if (a->q_dtype != expected_q_dtype(d.kv_dtype))
    return fail(PKV_E_DTYPE, "q_dtype must be f32 / f16 / bf16 for f32 / f16 / (bf16, fp8) pools");
  if (a->out_dtype != PKV_F32 && a->out_dtype != PKV_F16 && a->out_dtype != PKV_BF16)
    return fail(PKV_E_DTYPE, "out_dtype must be f32, f16 or bf16");
  if (!std::isfinite(a->scale)) return fail(PKV_E_INVAL, "scale must be finite");
  if (a->batch > 0 && (!a->q || !a->out || !a->context_lens || (a->max_blocks_per_seq > 0 && !a->block_tables)))
    return fail(PKV_E_INVAL, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->out)) % 16)
    return fail(PKV_E_INVAL, "q and out must be 16-byte aligned");
  if (a->shared_prefix_blocks < 0 || a->shared_prefix_blocks > a->max_blocks_per_seq)
    return fail(PKV_E_INVAL, "shared_prefix_blocks must lie in [0, max_blocks_per_seq]");
  if (a->shared_prefix_blocks > 0 && a->sliding_window > 0)
    return fail(PKV_E_UNSUPPORTED, "a shared prefix with a sliding window is not supported");
  if (a->new_k) {
    const bool same = a->new_dtype == d.kv_dtype;
    const bool quant = d.kv_dtype == PKV_FP8_E4M3 &&
                       (a->new_dtype == PKV_F32 || a->new_dtype == PKV_F16 || a->new_dtype == PKV_BF16);
    if (!same && !quant) return fail(PKV_E_DTYPE, "new_dtype must be the pool's dtype (or f32/f16/bf16 into FP8)");
    if (a->batch > 0 && (!a->new_v || !a->new_slots))
      return fail(PKV_E_INVAL, "a fused append needs new_k, new_v and new_slots");
    if ((reinterpret_cast<uintptr_t>(a->new_k) | reinterpret_cast<uintptr_t>(a->new_v)) % 16)
      return fail(PKV_E_INVAL, "new_k and new_v must be 16-byte aligned");
    if (a->batch > 0 && !a->block_tables)
      return fail(PKV_E_INVAL, "a fused append needs block_tables");
  } else if (a->new_v || a->new_slots) {
    return fail(PKV_E_INVAL, "new_v / new_slots given without new_k");
  }
  return PKV_OK;
}

// One pass per (KV head, sequence) with no merge: no shared prefix and a
// split count of 1 (or empty tables).
static bool single_pass(const paged_decode_args* a) {
  return a->shared_prefix_blocks == 0 && (a->num_splits == 1 || a->max_blocks_per_seq == 0);
}

// Every pair leaves a partial for the merge: with a shared prefix or a fused append.
static bool all_partial(const paged_decode_args* a) { return a->shared_prefix_blocks > 0 || a->new_k; }

static int tokens_per_subtile(int kv) {
  return kv == PKV_F32 ? SubTile<KV_F32>::TT : (kv == PKV_FP8_E4M3 ? SubTile<KV_FP8>::TT : SubTile<KV_BF16>::TT);
}

// Shared prefix work split: row groups (64 * NT query rows, one workgroup)
// per KV head and token chunks, about three workgroups per CU in all, at
// most 16 chunks.
static void prefix_plan(const kv_pool* pool, const paged_decode_args* a, int cus, int32_t* rtiles,
                        int32_t* chunks) {
  const kv_pool_desc& d = pool->desc;
  constexpr int rows_per_group = 4 * 16 * Decoder<KV_BF16, 128, 16>::NT;
  const int64_t G = a->num_q_heads / d.num_kv_heads;
  const int64_t rt = ((int64_t)a->batch * G + rows_per_group - 1) / rows_per_group;
  const int64_t tt = tokens_per_subtile(d.kv_dtype);
  const int64_t nsp = ((int64_t)a->shared_prefix_blocks * d.block_size + tt - 1) / tt;
  // three workgroups per CU: three wavefronts per SIMD (at most 168
  // registers each) hide each other's waits
  int64_t c = 3 * (int64_t)cus / std::max<int64_t>(1, d.num_kv_heads * rt);
  c = std::max<int64_t>(1, std::min<int64_t>({c, nsp, 16}));
  *rtiles = (int32_t)rt;
  *chunks = (int32_t)c;
}

static int64_t num_waves_for(const paged_decode_args* a, int cus) {
  return a->num_splits >= 2 ? (int64_t)a->num_splits : (int64_t)cus * kWavesPerCU;
}


// Workspace: merge jobs [Hkv][B] int4 (range mode, or every pair leaving a
// partial), partial outputs [W][2][G][D] fp32 and partial (max, sum)
// [W][2][G][2] fp32 (range mode), then, when every pair leaves a partial, the
// shared-prefix partials [chunks + 1][B * Hq][D + 4] fp32 (no chunks without
// a shared prefix; the last slot holds the own part of pairs that one
// wavefront held whole), and, with a fused append, the slots [B] int64; each
// part 256-byte aligned.
struct WsLayout {
  size_t job_off, o_off, ml_off, pre_off, slot_off, total;
};

static WsLayout workspace_layout(const kv_pool* pool, const paged_decode_args* a, int64_t W, bool single,
                                 int32_t pre_chunks) {
  const int64_t G = a->num_q_heads / pool->desc.num_kv_heads;
  auto up = [](size_t x) { return ((x + 255) / 256) * 256; };
  WsLayout l;
  l.job_off = l.o_off = l.ml_off = 0;
  size_t end = 0;
  if (!single || all_partial(a)) end = up((size_t)pool->desc.num_kv_heads * a->batch * sizeof(int4));
  if (!single) {
    l.o_off = end;
    l.ml_off = l.o_off + up((size_t)W * 2 * G * pool->desc.head_dim * sizeof(float));
    end = l.ml_off + up((size_t)W * 2 * G * 2 * sizeof(float));
  }
  l.pre_off = end;
  if (all_partial(a))
    end += up((size_t)(pre_chunks + 1) * a->batch * a->num_q_heads * (pool->desc.head_dim + 4) * sizeof(float));
  // fused append: the slots, as the append workgroups read them
  l.slot_off = end;
  if (a->new_k) end += up((size_t)a->batch * sizeof(int64_t));
  l.total = end;
  return l;
}

typedef void (*decode_fn)(DecodeParams);
typedef void (*tail_fn)(DecodeParams, TailParams);
typedef void (*prefix_fn)(DecodeParams);

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

template <int KV, int D>
static tail_fn pick_decode_append_bs(int bs) {
  switch (bs) {
    case 16: return decode_append_kernel<KV, D, 16>;
    case 32: return decode_append_kernel<KV, D, 32>;
    case 64: return decode_append_kernel<KV, D, 64>;
    case 128: return decode_append_kernel<KV, D, 128>;
  }
  return nullptr;
}

template <int KV>
static tail_fn pick_decode_append_d(int d, int bs) {
  return d == 64 ? pick_decode_append_bs<KV, 64>(bs) : pick_decode_append_bs<KV, 128>(bs);
}

// The decode that also stores a fused append's tokens (not for FP8 pools).
static tail_fn pick_decode_append(int kv, int d, int bs) {
  switch (kv) {
    case PKV_F32: return pick_decode_append_d<KV_F32>(d, bs);
    case PKV_F16: return pick_decode_append_d<KV_F16>(d, bs);
    case PKV_BF16: return pick_decode_append_d<KV_BF16>(d, bs);
  }
  return nullptr;
}

// The merge, compiled per (pool dtype, new-token dtype) for a fused append.
template <int D>
static tail_fn pick_merge(const DecodeParams& P) {
  if (!P.fused) return merge_kernel<D, -1, -1>;
  switch (P.kv_dtype) {
    case PKV_F32: return merge_kernel<D, KV_F32, KV_F32>;
    case PKV_F16: return merge_kernel<D, KV_F16, KV_F16>;
    case PKV_BF16: return merge_kernel<D, KV_BF16, KV_BF16>;
    default:
      if (P.new_src == PKV_F32) return merge_kernel<D, KV_FP8, KV_F32>;
      if (P.new_src == PKV_F16) return merge_kernel<D, KV_FP8, KV_F16>;
      return merge_kernel<D, KV_FP8, KV_BF16>;
  }
}

template <int KV, int D>
static prefix_fn pick_prefix_bs(int bs) {
  switch (bs) {
    case 16: return prefix_kernel<KV, D, 16>;
    case 32: return prefix_kernel<KV, D, 32>;
    case 64: return prefix_kernel<KV, D, 64>;
    case 128: return prefix_kernel<KV, D, 128>;
  }
  return nullptr;
}

static prefix_fn pick_prefix(int kv, int d, int bs) {
  switch (kv) {
    case PKV_F32: return d == 64 ? pick_prefix_bs<KV_F32, 64>(bs) : pick_prefix_bs<KV_F32, 128>(bs);
    case PKV_F16: return d == 64 ? pick_prefix_bs<KV_F16, 64>(bs) : pick_prefix_bs<KV_F16, 128>(bs);
    case PKV_BF16: return d == 64 ? pick_prefix_bs<KV_BF16, 64>(bs) : pick_prefix_bs<KV_BF16, 128>(bs);
    case PKV_FP8_E4M3: return d == 64 ? pick_prefix_bs<KV_FP8, 64>(bs) : pick_prefix_bs<KV_FP8, 128>(bs);
  }
  return nullptr;
}

// Workspace bytes of a decode call (arguments already checked).
static pkv_status workspace_bytes_for(const kv_pool* pool, const paged_decode_args* a, size_t* bytes_out) {
  const bool single = single_pass(a);
  int cus = 0;
  if ((!single && a->num_splits <= 1) || a->shared_prefix_blocks > 0) {
    const pkv_status st = device_cus(&cus);
    if (st != PKV_OK) return st;
  }
  int32_t rtiles = 0, chunks = 0;
  if (a->shared_prefix_blocks > 0) prefix_plan(pool, a, cus, &rtiles, &chunks);
  *bytes_out = workspace_layout(pool, a, single ? 0 : num_waves_for(a, cus), single, chunks).total;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// Static decode workspace, for callers that cannot allocate device memory.
// Every GPU the library runs on holds one copy of this array from the time
// the code object is loaded until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device array: its device address is
// looked up once per device with hipGetSymbolAddress and only that address
// is ever passed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[PKV_STATIC_WORKSPACE_BYTES];

static pkv_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices];   // per device, looked up on its first use
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_E_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PKV_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = p;
  }
  *out = addr[dev];
  return PKV_OK;
}

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

// [p, p + bytes) lies inside one HIP allocation of the wanted kind.
static bool in_one_allocation(const void* p, size_t bytes, hipMemoryType kind) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (at.type != kind) return false;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  return q >= b && bytes <= size && q - b <= size - bytes;
}

pkv_status pkv_hbm_read_probe(const void* d_buf, size_t bytes, uint32_t* d_sink, uint32_t tag,
                              pkv_stream stream) {
  if (bytes == 0) return PKV_OK;
  if (!d_buf || !d_sink) return fail(PKV_E_INVAL, "null pointer");
  if (reinterpret_cast<uintptr_t>(d_buf) % 16 || bytes % 16)
    return fail(PKV_E_INVAL, "buffer must be 16-byte aligned and bytes a multiple of 16");
  if (!in_one_allocation(d_buf, bytes, hipMemoryTypeDevice))
    return fail(PKV_E_INVAL, "buffer is not inside one device allocation");
  if (!in_one_allocation(d_sink, sizeof(uint32_t), hipMemoryTypeDevice))
    return fail(PKV_E_INVAL, "sink is not inside one device allocation");
  int cus = 0;
  pkv_status st = device_cus(&cus);
  if (st != PKV_OK) return st;
  const int64_t n16 = (int64_t)(bytes / 16);
  // 8 workgroups per CU, none with less than one round of loads
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(8 * (int64_t)cus, n16 / 1024));
  hipLaunchKernelGGL(read_probe_kernel, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(d_buf), n16, d_sink, tag);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : hip_fail(e, "read probe launch");
}

pkv_status kv_metadata_upload(void* d_dst, const void* h_src, size_t bytes, pkv_stream stream) {
  if (bytes == 0) return PKV_OK;
  if (!d_dst || !h_src) return fail(PKV_E_INVAL, "null pointer");
  if (reinterpret_cast<uintptr_t>(d_dst) % 8 || reinterpret_cast<uintptr_t>(h_src) % 8 || bytes % 4)
    return fail(PKV_E_INVAL, "src and dst must be 8-byte aligned and bytes a multiple of 4");
  if (!in_one_allocation(h_src, bytes, hipMemoryTypeHost))
    return fail(PKV_E_INVAL, "src is not inside one page-locked host allocation");
  if (!in_one_allocation(d_dst, bytes, hipMemoryTypeDevice))
    return fail(PKV_E_INVAL, "dst is not inside one device allocation");
  hipPointerAttribute_t at;
  hipError_t e = hipPointerGetAttributes(&at, h_src);
  if (e != hipSuccess || !at.devicePointer) return hip_fail(e, "hipPointerGetAttributes");
  const uint64_t* src = static_cast<const uint64_t*>(at.devicePointer);
  uint64_t* dst = static_cast<uint64_t*>(d_dst);
  const int64_t n8 = (int64_t)(bytes / 8);
  const uint32_t* src_tail = bytes % 8 ? reinterpret_cast<const uint32_t*>(src + n8) : nullptr;
  uint32_t* dst_tail = bytes % 8 ? reinterpret_cast<uint32_t*>(dst + n8) : nullptr;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n8 + 1023) / 1024, 1024));
  hipLaunchKernelGGL(upload_kernel, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream, src, dst, n8,
                     src_tail, dst_tail);
  e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : hip_fail(e, "upload launch");
}

static pkv_status append_launch(kv_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                int32_t src_dtype, const int64_t* d_slots, int32_t n_tokens, int32_t* d_tables,
                                int32_t* d_lens, int32_t max_blocks, pkv_stream stream) {
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
  P.tables = d_tables;
  P.lens = d_lens;
  P.max_blocks = max_blocks;
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

pkv_status paged_kv_append(kv_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                           int32_t src_dtype, const int64_t* d_slots, int32_t n_tokens,
                           pkv_stream stream) {
  return append_launch(pool, layer, d_k, d_v, src_dtype, d_slots, n_tokens, nullptr, nullptr, 0, stream);
}

pkv_status paged_kv_append_step(kv_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                int32_t src_dtype, const int64_t* slots, int32_t n, int32_t* d_tables,
                                int32_t* d_lens, int32_t max_blocks, pkv_stream stream) {
  if (n > 0 && (!d_tables || !d_lens || !slots)) return fail(PKV_E_INVAL, "null pointer");
  if (max_blocks <= 0) return fail(PKV_E_INVAL, "max_blocks must be positive");
  if (n <= 0) return n < 0 ? fail(PKV_E_INVAL, "bad argument") : PKV_OK;
  const size_t sb = (size_t)n * sizeof(int64_t);
  const int64_t* dev_slots = slots;
  if (in_one_allocation(slots, sb, hipMemoryTypeHost)) {
    hipPointerAttribute_t at;
    hipError_t e = hipPointerGetAttributes(&at, slots);
    if (e != hipSuccess || !at.devicePointer) return hip_fail(e, "hipPointerGetAttributes");
    dev_slots = static_cast<const int64_t*>(at.devicePointer);
  } else if (!in_one_allocation(slots, sb, hipMemoryTypeDevice)) {
    return fail(PKV_E_INVAL, "slots must lie in one device or page-locked host allocation");
  }
  if (!in_one_allocation(d_tables, (size_t)n * max_blocks * sizeof(int32_t), hipMemoryTypeDevice) ||
      !in_one_allocation(d_lens, (size_t)n * sizeof(int32_t), hipMemoryTypeDevice))
    return fail(PKV_E_INVAL, "tables and lengths must lie in device allocations of [n][max_blocks] and [n]");
  return append_launch(pool, layer, d_k, d_v, src_dtype, dev_slots, n, d_tables, d_lens, max_blocks, stream);
}

pkv_status paged_attention_workspace_size(const kv_pool* pool, const paged_decode_args* a, size_t* bytes_out) {
  if (!bytes_out) return fail(PKV_E_INVAL, "null argument");
  pkv_status st = check_decode(pool, a);
  if (st != PKV_OK) return st;
  return workspace_bytes_for(pool, a, bytes_out);
}

}  // extern "C"

// Launch on s; start / stop (may be NULL) record when the first kernel
// starts and the last one ends.
template <typename K, typename... Args>
static hipError_t launch(K kernel, dim3 grid, size_t lds, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                         Args... args) {
  if (start || stop) hipExtLaunchKernelGGL(kernel, grid, dim3(256), (uint32_t)lds, s, start, stop, 0u, args...);
  else hipLaunchKernelGGL(kernel, grid, dim3(256), lds, s, args...);
  return hipGetLastError();
}

// ev: NULL or {attention start, attention end, merge start, merge end};
// *nk: kernels launched.
static pkv_status decode_launch(const kv_pool* pool, const paged_decode_args* a, pkv_stream stream,
                                hipEvent_t const* ev, int32_t* nk) {
  if (nk) *nk = 0;
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
  P.ws_job = nullptr;
  P.ws_pre = nullptr;
  P.xcd_remap = 0;
  P.nstage = 0;
  P.stage_off = 0;
  P.lens_in_lds = 0;
  P.shared = a->shared_prefix_blocks;
  P.pre_chunks = 0;
  P.pre_rtiles = 0;
  P.allpart = all_partial(a) ? 1 : 0;
  P.fused = a->new_k ? 1 : 0;
  P.new_src = a->new_dtype;
  P.kv_dtype = d.kv_dtype;
  P.block_size = d.block_size;
  P.new_k = (const uint8_t*)a->new_k;
  P.new_v = (const uint8_t*)a->new_v;
  P.new_slots = a->new_slots;
  P.k_inv = d.k_inv_scale;
  P.v_inv = d.v_inv_scale;
  P.tables_w = a->block_tables;
  P.lens_w = a->context_lens;
  P.merge_pg = 1;
  P.append_spg = append_seqs_per_group(d.num_kv_heads, d.head_dim, d.kv_dtype);
  TailParams TP;
  TP.decode_wgs = 0;
  TP.ws_slots = nullptr;
  if (P.fused) {
    // the slots may be in page-locked host memory (the host block manager's
    // buffer): the merge then reads them through its device address
    const size_t sb = (size_t)a->batch * sizeof(int64_t);
    if (in_one_allocation(a->new_slots, sb, hipMemoryTypeHost)) {
      hipPointerAttribute_t at;
      const hipError_t e = hipPointerGetAttributes(&at, a->new_slots);
      if (e != hipSuccess || !at.devicePointer) return hip_fail(e, "hipPointerGetAttributes");
      P.new_slots = static_cast<const int64_t*>(at.devicePointer);
    } else if (!in_one_allocation(a->new_slots, sb, hipMemoryTypeDevice)) {
      return fail(PKV_E_INVAL, "new_slots must lie in one device or page-locked host allocation of [batch]");
    }
  }
  decode_fn fn = pick_decode(d.kv_dtype, d.head_dim, d.block_size);
  if (!fn) return fail(PKV_E_UNSUPPORTED, "no kernel for this shape");
  // fused append into a pool other than FP8: the decode's tail stores the tokens
  const tail_fn afn =
      P.fused && d.kv_dtype != PKV_FP8_E4M3 ? pick_decode_append(d.kv_dtype, d.head_dim, d.block_size) : nullptr;
  if (P.fused && d.kv_dtype != PKV_FP8_E4M3 && !afn) return fail(PKV_E_UNSUPPORTED, "no kernel for this shape");
  hipStream_t s = (hipStream_t)stream;
  const int64_t segs = (int64_t)d.num_kv_heads * a->batch;
  // a shared prefix always runs in range mode (its merge joins the prefix)
  const bool single = single_pass(a);

  int cus = 0;
  if ((!single && a->num_splits <= 1) || P.shared > 0) {
    st = device_cus(&cus);
    if (st != PKV_OK) return st;
  }
  const int64_t W = single ? 0 : num_waves_for(a, cus);
  if (P.shared > 0) prefix_plan(pool, a, cus, &P.pre_rtiles, &P.pre_chunks);
  const WsLayout wl = workspace_layout(pool, a, W, single, P.pre_chunks);
  char* ws = reinterpret_cast<char*>(a->workspace);
  if (wl.total > 0) {
    if (!a->workspace || a->workspace_bytes < wl.total)
      return fail(PKV_E_INVAL, "workspace missing or smaller than paged_attention_workspace_size()");
    if (reinterpret_cast<uintptr_t>(a->workspace) % 256)
      return fail(PKV_E_INVAL, "workspace must be 256-byte aligned");
  }
  // the first kernel launched records ev[0]
  hipEvent_t ev_first = ev ? ev[0] : nullptr;
  hipError_t e;
  if (P.allpart) P.ws_pre = reinterpret_cast<float*>(ws + wl.pre_off);
  if (P.fused) TP.ws_slots = reinterpret_cast<int64_t*>(ws + wl.slot_off);
  // fused append: the token-storing workgroups after the decode's (FP8:
  // merge_kernel stores them)
  const int64_t nappend =
      P.fused && d.kv_dtype != PKV_FP8_E4M3 ? (a->batch + P.append_spg - 1) / P.append_spg : 0;
  if (P.shared > 0) {
    prefix_fn pfn = pick_prefix(d.kv_dtype, d.head_dim, d.block_size);
    if (!pfn) return fail(PKV_E_UNSUPPORTED, "no kernel for this shape");
    const int64_t tasks = (int64_t)d.num_kv_heads * P.pre_rtiles * P.pre_chunks;
    const int64_t pgrid = ((tasks + 7) / 8) * 8;  // one workgroup per task, whole rounds over the 8 XCDs
    e = launch(pfn, dim3((uint32_t)pgrid), 0, s, ev_first, nullptr, P);
    if (e != hipSuccess) return hip_fail(e, "prefix launch");
    ev_first = nullptr;
  }

  const tail_fn mfn = d.head_dim == 64 ? pick_merge<64>(P) : pick_merge<128>(P);
  if (single) {
    P.single = 1;
    P.num_waves = 0;
    if (P.allpart) P.ws_job = reinterpret_cast<int4*>(ws + wl.job_off);
    const int64_t grid = (segs + 3) / 4;
    TP.decode_wgs = (int32_t)grid;
    e = afn ? launch(afn, dim3((uint32_t)(grid + nappend)), 0, s, ev_first, ev ? ev[1] : nullptr, P, TP)
            : launch(fn, dim3((uint32_t)grid), 0, s, ev_first, ev ? ev[1] : nullptr, P);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    if (nk) *nk = 1;
    if (!P.fused) return PKV_OK;
    // the fused append's merge: every pair's own partial and the new token,
    // and the workgroups that write the rows' tables and lengths
    P.merge_pg = 1;
    const int64_t mgrid = segs + (merge_row_groups(P) + 7) / 8 * 8;
    e = launch(mfn, dim3((uint32_t)mgrid), 0, s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, P, TP);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    if (nk) *nk = 2;
    return PKV_OK;
  }

  P.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
  P.ws_ml = reinterpret_cast<float*>(ws + wl.ml_off);
  P.ws_job = reinterpret_cast<int4*>(ws + wl.job_off);
  P.single = 0;
  P.num_waves = (int32_t)W;
  int64_t grid = (W + 3) / 4;
  grid = ((grid + 7) / 8) * 8;  // whole rounds over the 8 XCDs
  P.xcd_remap = 1;
  // unit prefix sums (and, up to 4096 sequences, the context lengths), then
  // as many staging slots per wavefront (at most 4) as fit, with the static
  // LDS, in 64 KiB
  P.lens_in_lds = a->batch <= 4096 ? 1 : 0;
  P.stage_off = (int32_t)(((a->batch + 1 + (P.lens_in_lds ? a->batch : 0)) * (int64_t)sizeof(int32_t) + 15) / 16 * 16);
  const int64_t per_slot = 4 * (int64_t)(4 * P.group * (d.head_dim + 8) + (int64_t)sizeof(PieceTag));
  P.nstage = (int32_t)std::max<int64_t>(0, std::min<int64_t>(4, (63488 - P.stage_off) / per_slot));
  const size_t lds = (size_t)P.stage_off + (size_t)P.nstage * per_slot;
  TP.decode_wgs = (int32_t)grid;
  e = afn ? launch(afn, dim3((uint32_t)(grid + nappend)), lds, s, ev_first, ev ? ev[1] : nullptr, P, TP)
          : launch(fn, dim3((uint32_t)grid), lds, s, ev_first, ev ? ev[1] : nullptr, P);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (nk) *nk = 1;
  // few sequence-heads: spread each one's output positions over several
  // workgroups so that the merge still uses most CUs
  const int np = (int)(P.group * (d.head_dim / 4));
  int pg = 1;
  while (segs * pg < 512 && np / (pg * 2) >= 16) pg *= 2;
  P.merge_pg = pg;
  const int64_t mgrid = segs * pg + (P.fused ? (merge_row_groups(P) + 7) / 8 * 8 : 0);
  e = launch(mfn, dim3((uint32_t)mgrid), 0, s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, P, TP);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  if (nk) *nk = 2;
  return PKV_OK;
}

extern "C" {

pkv_status paged_attention_decode(const kv_pool* pool, const paged_decode_args* a, pkv_stream stream) {
  return decode_launch(pool, a, stream, nullptr, nullptr);
}

pkv_status paged_attention_decode_static(const kv_pool* pool, const paged_decode_args* a, pkv_stream stream) {
  pkv_status st = check_decode(pool, a);
  if (st != PKV_OK) return st;
  if (a->workspace || a->workspace_bytes)
    return fail(PKV_E_INVAL, "paged_attention_decode_static uses the library's static workspace: "
                             "workspace must be NULL and workspace_bytes 0");
  size_t need = 0;
  st = workspace_bytes_for(pool, a, &need);
  if (st != PKV_OK) return st;
  if (need > PKV_STATIC_WORKSPACE_BYTES)
    return fail(PKV_E_UNSUPPORTED, "this call needs " + std::to_string(need) +
                                       " bytes of workspace, more than the static workspace's " +
                                       std::to_string((size_t)PKV_STATIC_WORKSPACE_BYTES) +
                                       ": use paged_attention_decode with a caller-owned workspace");
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  // the decode rewrites every workspace record it reads on each call, so the
  // previous call's contents need no clearing
  paged_decode_args c = *a;
  c.workspace = ws;
  c.workspace_bytes = PKV_STATIC_WORKSPACE_BYTES;
  return decode_launch(pool, &c, stream, nullptr, nullptr);
}

pkv_status paged_attention_decode_timed(const kv_pool* pool, const paged_decode_args* a, pkv_stream stream,
                                        void* const* kernel_events, int32_t* n_kernels_out) {
  if (!kernel_events) return fail(PKV_E_INVAL, "kernel_events is NULL");
  for (int k = 0; k < 4; ++k)
    if (!kernel_events[k]) return fail(PKV_E_INVAL, "kernel_events needs four events");
  return decode_launch(pool, a, stream, reinterpret_cast<hipEvent_t const*>(kernel_events), n_kernels_out);
}

}  // extern "C"
