// Split-KV low-bit MLA decode for groups of 16 query heads on gfx950 (CDNA4).
//
// Same computation as decode64.hip (QuantMLA pages: ai.info summary, "Key
// Contributions", item 4; onedev.kr review, "How it is used"): one global
// softmax over all valid tokens, sink / recent tokens from bf16, all others
// from their packed copies, output aggregated over the content latent.
//
// With 16 heads per latent the decode is HBM-bound: every packed code feeds a
// single 16-head MFMA block.  One workgroup of 8 waves (two per SIMD) per
// (work item, 16-head group), working as four independent pairs: pair r is
// waves r and r + 4, on one SIMD, splitting the work by role and running
// concurrently, so one wave's stalls are covered by the other's work.  The two
// hand blocks over through LDS sequence flags in a two-buffer ring.
//
// Packed items (the quantized middle of a sequence) go in 32-token blocks,
// half a page each, pair r taking blocks r, r + 4, ...:
//  - the PV wave loads a block's content words one block ahead with
//    contiguous 16-byte loads, writes the codes to the pair's tile as one byte
//    per code, and for every block the QK wave has scored accumulates MFMA
//    16x16x32 f16 of the codes (8-bit transposed LDS reads, widened exactly to
//    fp16 subnormals)
//    against p * s_g, plus the zero terms sum_t p_t z_g,t;
//  - the QK wave multiplies the tile's code bytes by the query with MFMA
//    16x16x64 i8: the query in fixed point, three int8 digits per component,
//    so each group's product is an exact integer, then the token's fp32 group
//    scale; the RoPE-key codes and the metadata words it loads itself; the
//    zero terms of all nine groups through one f16 MFMA; online softmax in the
//    log2 domain with a lazily refreshed running max; the fp16 probabilities,
//    PV scales and zeros go to the pair's tile.
// bf16 items (the sink and recent tokens) go in 16-token
// blocks: the QK wave loads the rows, multiplies them in fp16 (MFMA 16x16x32,
// the query as the A operand) and writes them to the tile for the PV wave.
// Every wait is bounded, so a broken handshake gives wrong values, never a
// hang; a wait that gives up is counted in the workspace header.  The four
// pairs' partials are merged through LDS at the end; the item's partial stays
// unnormalised with its running max and sum for the combine.
#include <algorithm>
#include <cstddef>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

constexpr int kPairs = 4;             // QK waves 0..3, PV waves 4..7 (pair r: waves r and r + 4)
constexpr int kThreads = 128 * kPairs;
constexpr int kB = 16;                // tokens per block (one pair's rows of a page)
constexpr int kSV = 528;              // V tile row stride (halves): conflict-free b128 row writes and transposed reads
constexpr int kPS = 16;               // probability / zero row stride (halves), rows are tokens
constexpr float kRescale = 8.0f;      // lazy max refresh threshold, log2 units

template <int BITS_C>
struct Geo {
  static constexpr int CB = kDc * BITS_C / 8;                              // content bytes per token
  static constexpr int PB = kPageTokens * (CB + kDr / 2 + 4 * kGroups);   // page bytes
  static constexpr int ROPE0 = kPageTokens * CB;
  static constexpr int META0 = kPageTokens * (CB + kDr / 2);
};

// A pair's tiles for one block: written by its QK wave, read by its PV wave (two buffers a pair:
// blocks t and t + 1).
struct __align__(16) PairTiles {
  f16 V[kB][kSV];     // exact content codes of the block [token][channel position]
  f16 P[kB][kPS];     // fp16 probabilities [token][head]
  f16 Z[kB][kPS];     // fp16 zeros [token][z_0..z_7, z_8, 0 x 7]
  f16 SV[8][kB];      // fp16 PV group scales [group][token]
  float alpha[16];    // per-head factor for the PV accumulators before this block (running max refreshed)
  int resc;           // 1: apply alpha before this block
  int pad[3];
};
struct MergeArea {          // merge of the pairs' partials at the end (two pairs at a time)
  float o[2][16][kDc];
  float m[kPairs][16], l[kPairs][16];
  float z[kPairs][16][8];
};

// Packed items run in 32-token blocks (half a page) whose codes sit in LDS one byte each: code c
// (0..15) is the byte c (the int8 c to the QK MFMA; zero-extended to 16 bits, the fp16 c * 2^-24
// to the PV MFMA, whose sums are scaled back by 2^24 at the end).  A token row holds 32 units of 16 code bytes; unit u covers the 16 channels from pk_unit_base(u) on, byte b of it channel
// pk_unit_base(u) + pk_unit_off(b), an order that lets the unpacking write whole units and lets
// both multiplications read them directly.
constexpr int kPB = 32;    // tokens per packed block
constexpr int kVS = 528;   // code tile row stride (bytes): 33 units of 16, odd, so the same unit of
                           // 16 consecutive rows falls in distinct banks
// Row strides of the small per-block buffers, chosen for the LDS banks: the QK wave's 8-byte
// probability writes (16 token rows per pass) and 2-byte scale / zero writes cover distinct banks.
constexpr int kPkP = 20;   // probability row stride (halves)
constexpr int kPkS = 48;   // PV scale / zero row stride (halves)
struct __align__(16) PkBuf {
  uint8_t V[kPB][kVS];     // code bytes [token][unit order]
  f16 P[kPB][kPkP];        // fp16 probabilities [token][head]
  f16 SV[8][kPkS];         // PV scales s_g * 2^-E [group][token]; 0 for masked tokens
  f16 Z[8][kPkS];          // zeros z_g [group][token]; 0 for masked tokens
  float alpha[16];         // per-head factor for the PV accumulators before this block
  int resc;                // bit 0: apply alpha before this block; bit 1: the PV scale exponent changed
  int pv_exp;              // E: the block's PV scales are fp16(s * 2^-E) (valid with bit 1 of resc)
  int pad[2];
};
constexpr int kDigits = 3;  // base-128 digits of a query component's fixed-point value
struct __align__(16) PkPrologue {  // before the first block: the query digits, built once per workgroup
  uint32_t A[kGroups][kDigits][64][4];  // QK lanes' A operands (16 int8 digits a lane, group and digit)
  float amax[16][36];              // per head: partial max |q| of its 36 spans of 16 channels
  float qsum[16][kGroups][4];      // per head and group: partial sums of q over 16 channels
  int hk[16];                      // per head: the power of two applied before rounding
};

union __align__(16) Tiles16 {
  PairTiles pt[kPairs][2];   // bf16 items
  PkBuf pk[kPairs][2];       // packed items
  PkPrologue pro;
  MergeArea mg;
};

__device__ __forceinline__ f32x4 mfma32k(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// (max: DPP within the row, lanes i ^ 1 and i ^ 2 (quad_perm), then the mirrored lane of the half
// row and of the row; every lane ends with the row's maximum, and no LDS round trip is taken)
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_row<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_row<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_row<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_row<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  return v + __shfl_xor(v, 8, 64);
}


// ---- merge of the four pairs' partials, shared by both item kinds.  The QK wave of pair pr gives
// its running maxima and sums; the PV wave brings its accumulators to the merged maximum (and
// multiplies them by 2^cur_e, undoing the PV scale normaliser and the codes' operand scale), the
// pairs' outputs are summed through LDS into pair 0, which passes them to write() and stores the
// running max, sum and the zero-term sums of the split's row.  When the item is its sequence's only
// one (direct), pair 0 instead has write() store the final bf16 outputs (sum plus the group's zero
// term, over the sum of probabilities) and stores the lse, as the combine would.  Both roles pass
// five workgroup barriers.
__device__ __forceinline__ void merge_qk(MergeArea& mg, const float (&m_run)[4], const float (&l_part)[4], int pr,
                                         int G, int L16) {
  __syncthreads();  // every wave is done with its tiles; the merge area overlays them
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l_row = row16_sum(l_part[i]);
    if (L16 == 0) {
      mg.m[pr][4 * G + i] = m_run[i];
      mg.l[pr][4 * G + i] = l_row;
    }
  }
  __syncthreads();
  __syncthreads();
  __syncthreads();
  __syncthreads();
}

template <typename Write>
__device__ __forceinline__ void merge_pv(const DecodeParams& p, MergeArea& mg, f32x4 (&O)[32], f32x4 oz, int cur_e,
                                         int pr, int lane, int G, int L16, int64_t orow, bool direct,
                                         int64_t out_row, Write write) {
  __syncthreads();  // every wave is done with its tiles; the merge area overlays them
  __syncthreads();  // the QK waves' running maxima and sums are in place
  float M = -__builtin_inff();  // merged max of head L16 (the PV column)
#pragma unroll
  for (int v = 0; v < kPairs; ++v) M = fmaxf(M, mg.m[v][L16]);
  {
    const float mw = mg.m[pr][L16];
    const float f = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    const float fe = __builtin_ldexpf(f, cur_e);  // undo the PV scale normaliser (f <= 1)
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) O[cb] *= fe;
    oz *= f;
  }
  if (G < 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mg.z[pr][L16][4 * G + i] = oz[i];
  }
  // pairs 2, 3 hand their outputs to pairs 0, 1; then pair 1 hands the sum to pair 0.  Every
  // PV wave holds the same (head, channel) in the same lane and register, so the hand-over area
  // is laid out as the registers are: [register][lane], 16 bytes a lane, no bank conflicts.
  auto put = [&](int k) {
    const lds_ptr<f32x4> o4 = (lds_ptr<f32x4>)&mg.o[k][0][0];
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) o4[64 * cb + lane] = O[cb];
  };
  auto add = [&](int k) {
    const lds_ptr<f32x4> o4 = (lds_ptr<f32x4>)&mg.o[k][0][0];
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) O[cb] += o4[64 * cb + lane];
  };
  if (pr >= 2) put(pr - 2);
  __syncthreads();
  if (pr < 2) add(pr);
  __syncthreads();
  if (pr == 1) put(0);
  __syncthreads();
  if (pr == 0) {
    add(0);
    float L = 0.f, zs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // of head L16
#pragma unroll
    for (int v = 0; v < kPairs; ++v) {
      const float mv = mg.m[v][L16];
      L += (mv == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mv - M)) * mg.l[v][L16];
#pragma unroll
      for (int g = 0; g < 8; ++g) zs[g] += mg.z[v][L16][g];
    }
    if (direct) {
      write(O, zs, M == -__builtin_inff() ? 0.f : 1.f / L);
      if (G == 0 && p.lse)
        p.lse[out_row] = M == -__builtin_inff() ? -__builtin_inff() : (M + __log2f(L)) * 0.69314718055994531f;
    } else {
      write(O, zs, 0.f);
      if (G == 0) {
        p.ws_ml[2 * orow] = M;
        p.ws_ml[2 * orow + 1] = L;
#pragma unroll
        for (int g = 0; g < 8; ++g) p.ws_z[orow * 8 + g] = zs[g];
      }
    }
  }
}

// ---- packed items
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

// first channel of unit u's 16-channel span, and the channel offset of its byte b (RoPE-key bytes
// follow the 4-bit order)
template <int BITS_C>
__device__ __forceinline__ constexpr int pk_unit_base(int u) {
  return BITS_C == 4 ? (u < 16 ? 32 * u : 32 * (u - 16) + 16) : 64 * (u & 7) + 16 * (u >> 3);
}
template <int BITS_C>
__device__ __forceinline__ constexpr int pk_unit_off(int b) {
  return BITS_C == 4 ? 8 * (b >> 3) + 2 * (b & 3) + ((b >> 2) & 1) : 4 * (b & 3) + (b >> 2);
}
// the four units of group g (g < 8): unit qk_unit(g, q) is the one QK lanes 16 q .. 16 q + 15 multiply.
// Lane groups q = 0, 1 (and 2, 3) share the passes of a 16-byte LDS read; their units lie 16 apart,
// i.e. 64 dwords, so that with the 132-dword row stride the 16 rows of both fall on distinct banks.
template <int BITS_C>
__device__ __forceinline__ constexpr int qk_unit(int g, int q) {
  return BITS_C == 4 ? 16 * (q & 1) + 2 * g + (q >> 1) : 16 * (q & 1) + 8 * (q >> 1) + g;
}

// 8 nibbles -> 8 code bytes (channels 0 2 4 6 | 1 3 5 7 of the dword)
__device__ __forceinline__ void nib_bytes(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = w & 0x0F0F0F0Fu;
  hi = (w >> 4) & 0x0F0F0F0Fu;
}

// Exact integer product of a group's 64 query components (fixed point, three base-128 int8 digits
// d0 d1 d2, value 2^14 d0 + 2^7 d1 + d2) with its 64 code bytes: each MFMA 16x16x64 i8 adds one
// digit's products to the accumulator after the shift by 7 bits, so the chain ends with the whole
// fixed-point product (|value| <= 2^20, codes <= 15: at most 2^30 in magnitude, no overflow).
// Two such chains (two 16-token halves) side by side, so one's shift overlaps the other's MFMA.
__device__ __forceinline__ void qk_group2(const i32x4 (&a)[kDigits], const i32x4 (&b)[2], i32x4 (&x)[2]) {
  x[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[0], i32x4{0, 0, 0, 0}, 0, 0, 0);
  x[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[1], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
  for (int j = 1; j < kDigits; ++j) {
    x[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b[0], x[0] << 7, 0, 0, 0);
    x[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b[1], x[1] << 7, 0, 0, 0);
  }
}
__device__ __forceinline__ f32x4 to_f32x4(i32x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 mfma32k_acc(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 code bytes (a tr_b8 column: 8 tokens of one channel) -> 8 fp16 operands: each byte c (c <= 15)
// zero-extended to 16 bits, the fp16 subnormal c * 2^-24 exactly (one byte permute per two codes).
// The MFMA keeps fewer bits of products with subnormal operands (relative error about 2^-18 of the
// summed magnitudes instead of 2^-24), ample for the PV sums but not for the scores.
__device__ __forceinline__ f16x8 codes_to_f16(u32x2 v) {
  const uint32_t a = __builtin_amdgcn_perm(0u, v.x, 0x0c010c00u), b = __builtin_amdgcn_perm(0u, v.x, 0x0c030c02u);
  const uint32_t c = __builtin_amdgcn_perm(0u, v.y, 0x0c010c00u), d = __builtin_amdgcn_perm(0u, v.y, 0x0c030c02u);
  return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}

struct ItemCtx {
  int item, b, slot, p_lo, p_hi, page0, n_pages, head0;
};

// One packed item (pages page0 .. page0 + n_pages - 1 of the sequence), 16 heads.  Pair pr (waves
// pr and pr + 4, one SIMD) takes the item's 32-token blocks pr, pr + 4, ... in page order:
//  - the PV wave (pr + 4) loads a block's content codes with contiguous 16-byte loads one block
//    ahead, turns them into code bytes and writes them to the pair's code tile; for every block
//    the QK wave has scored it accumulates MFMA 16x16x32 f16 of the codes (8-bit transposed LDS
//    reads, widened to fp16 subnormals c * 2^-24) against p * s_g * 2^-E, and the zero-term sums;
//  - the QK wave (pr) multiplies the tile's code bytes by the queries with MFMA 16x16x64 i8: each
//    head's query, times a power of two that puts its largest component in [2^19, 2^20), is rounded
//    to an integer (exact for every component above 2^-12 of the largest, which bf16 holds with 8
//    significant bits) and split into three int8 digits, so every group's product is an exact
//    integer; the RoPE-key codes it loads and unpacks itself; fp32 group scales per token, zero
//    terms through one f16 MFMA, online softmax; it writes the probabilities, PV scales and zeros
//    to the pair's buffer.
// Flags: s_flag[pr][0] = last block whose probabilities are published (QK -> PV), s_flag[pr][1] =
// last block whose codes are in the tile (PV -> QK).  The PV wave writes block t + 2 into buffer
// t % 2 once it has finished block t, whose probabilities the QK wave published after scoring it.
template <int BITS_C>
__device__ __forceinline__ void packed_item(const DecodeParams& p, Tiles16& s_tiles, int (&s_flag)[kPairs][4],
                                            const ItemCtx& it) {
  constexpr int CB = kDc * BITS_C / 8;                             // content bytes per token
  constexpr int PGB = kPageTokens * (CB + kDr / 2 + 4 * kGroups);  // page bytes
  constexpr int ROPE0 = kPageTokens * CB, META0 = kPageTokens * (CB + kDr / 2);
  constexpr int NLD = kPB * CB / 1024;  // 16-byte content loads per PV lane and block (4-bit: 8, 2-bit: 4)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = w & (kPairs - 1);
  const int G = lane >> 4, L16 = lane & 15;
  const int n_blk = 2 * it.n_pages;
  const int nb = n_blk > pr ? (n_blk - pr + kPairs - 1) / kPairs : 0;  // this pair's blocks
  const float c_log2 = p.scale_log2e;
  const int spin = p.spin_limit;
  typedef __attribute__((address_space(4))) const int32_t cint;
  cint* bt = (cint*)(uintptr_t)(p.block_table + (int64_t)it.slot * p.max_pages + it.page0);
  lds_vint* const fl = (lds_vint*)&s_flag[pr][0];
  // page of the pair's block t (clamped to its last block; nb > 0): block j = pr + 4 t is half
  // j % 2 of page j / 2 of the item; an id outside the pool reads page 0 and is counted
  auto page_ptr = [&](int t, int& bad) -> const uint8_t* {
    const int j = pr + kPairs * min(t, nb - 1);
    int pg = bt[j >> 1];
    if (pg < 0 || pg >= p.num_pages) {
      pg = 0;
      ++bad;
    }
    return p.pages + (int64_t)pg * PGB;
  };
  int give_ups = 0, bad_pages = 0;

  // ---- query digits (all 512 threads).  Task (g, hh, q): the 16 channels of group g that QK lane
  // 16 q + hh multiplies (unit qk_unit(g, q) for g < 8; RoPE-key channels 16 q .. 16 q + 15 for
  // g = 8, in the 4-bit byte order); byte b of the lane's operand is channel base + unit_off(b).
  PkPrologue& pro = s_tiles.pro;
  {
    float v[2][16];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int task = tid + 512 * k;
      if (task < kGroups * 64) {
        const int g = task >> 6, hh = (task >> 2) & 15, q = task & 3;
        const int base = g < 8 ? pk_unit_base<BITS_C>(qk_unit<BITS_C>(g, q)) : kDc + 16 * q;
        const uint4* src = reinterpret_cast<const uint4*>(p.q + ((int64_t)it.b * p.heads + it.head0 + hh) * kD + base);
        const uint4 r0 = src[0], r1 = src[1];
        const uint32_t wd[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        float mx = 0.f, sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[k][i] = bf16f((i & 1) ? (wd[i >> 1] >> 16) : (wd[i >> 1] & 0xFFFFu));
          mx = fmaxf(mx, fabsf(v[k][i]));
          sum += v[k][i];
        }
        pro.amax[hh][4 * g + q] = mx;
        pro.qsum[hh][g][q] = sum;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int task = tid + 512 * k;
      if (task < kGroups * 64) {
        const int g = task >> 6, hh = (task >> 2) & 15, q = task & 3;
        float mx = 0.f;
        for (int i = 0; i < 36; ++i) mx = fmaxf(mx, pro.amax[hh][i]);
        // fixed point: the largest component scaled into [2^19, 2^20) (a head whose largest
        // component is below 2^-45 keeps the scale 2^64)
        const int hk = mx > 0.f ? min(19 - (((__float_as_int(mx) >> 23) & 0xFF) - 127), 64) : 0;
        if (task < 64 && (task & 3) == 0) pro.hk[hh] = hk;  // one task of each head (g = 0)
        const float sc = __builtin_ldexpf(1.f, hk);
        uint32_t dg[kDigits][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int j = 0; j < kDigits; ++j) dg[j][d] = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int bb = 4 * d + e;
            const int off = (g == 8 || BITS_C == 4) ? pk_unit_off<4>(bb) : pk_unit_off<2>(bb);
            // value = 2^14 d0 + 2^7 d1 + d2 with d1, d2 in [-64, 63] and |d0| <= 64
            const int x = (int)__builtin_rintf(v[k][off] * sc);
            const int d2 = ((x + 64) & 127) - 64;
            const int x1 = (x - d2) >> 7;
            const int d1 = ((x1 + 64) & 127) - 64;
            const int d0 = (x1 - d1) >> 7;
            dg[0][d] |= (uint32_t)(d0 & 0xFF) << (8 * e);
            dg[1][d] |= (uint32_t)(d1 & 0xFF) << (8 * e);
            dg[2][d] |= (uint32_t)(d2 & 0xFF) << (8 * e);
          }
        }
#pragma unroll
        for (int j = 0; j < kDigits; ++j)
          *reinterpret_cast<uint4*>(&pro.A[g][j][16 * q + hh][0]) = make_uint4(dg[j][0], dg[j][1], dg[j][2], dg[j][3]);
      }
    }
    __syncthreads();
  }

  if (w < kPairs) {
    // ================================ QK wave of pair pr ================================
    i32x4 qa[kGroups][kDigits];
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int j = 0; j < kDigits; ++j) {
        const uint4 a = *reinterpret_cast<const uint4*>(&pro.A[g][j][lane][0]);
        qa[g][j] = i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
      }
    f16x8 qz;  // zero-term A operand: k = 8 G + j: G0 hi(qs_j), G1 lo(qs_j), G2 / G3 hi / lo of qs_8 at j = 0
    {
      float qs[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        qs[g] = (pro.qsum[L16][g][0] + pro.qsum[L16][g][1] + pro.qsum[L16][g][2] + pro.qsum[L16][g][3]) * c_log2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = G < 2 ? qs[j] : (j == 0 ? qs[8] : 0.f);
        const f16 hi = (f16)x;
        const f16 lo = (f16)(x - (float)hi);
        qz[j] = (G & 1) ? lo : hi;
      }
    }
    f32x4 hs;  // per output row (head 4 G + i): scale * log2 e * 2^-hk
#pragma unroll
    for (int i = 0; i < 4; ++i) hs[i] = __builtin_ldexpf(c_log2, -pro.hk[4 * G + i]);
    __syncthreads();  // the prologue area is read; the buffers overlay it from here on

    float m_run[4], l_part[4];  // heads 4G + i
    float m_thr[4], m_sub[4];   // m_run + kRescale, and m_run as subtracted from scores (0 while -inf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_thr[i] = -__builtin_inff();
      m_sub[i] = 0.f;
      m_run[i] = -__builtin_inff();
      l_part[i] = 0.f;
    }
    int pv_e = 0;
    float pv_inv = 1.f, pv_hi = 0x1p-126f;  // PV scale normaliser (raised when a scale reaches pv_hi)

    // per block: the lane's RoPE-key codes (8 packed bytes, channels 16 G .. 16 G + 15, of each of
    // its two tokens) and the nine metadata words of its two tokens
    struct QRegs {
      uint2 r[2];
      uint32_t m[2][kGroups];
    };
    auto qload = [&](int t, QRegs& R) {
      const uint8_t* base = page_ptr(t, bad_pages);
      const int half = (pr + kPairs * min(t, nb - 1)) & 1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 32 * half + 16 * h + L16;
        R.r[h] = *reinterpret_cast<const uint2*>(base + ROPE0 + row * (kDr / 2) + 8 * G);
        const uint32_t* mrow = reinterpret_cast<const uint32_t*>(base + META0 + row * 4 * kGroups);
#pragma unroll
        for (int g = 0; g < kGroups; ++g) R.m[h][g] = mrow[g];
      }
    };
    auto qblock = [&](int t, const QRegs& R) {
      const int j = pr + kPairs * t;
      const int tok0 = (it.page0 + (j >> 1)) * kPageTokens + (j & 1) * kPB;
      PkBuf& B = s_tiles.pk[pr][t & 1];
      const lds_ptr<uint8_t> vb = lds_opaque(&B.V[0][0]);
      give_ups += wait_at_least(fl + 1, t, spin);  // block t's codes are in the tile
      f32x4 S[2];
      uint32_t mw[2][kGroups];
      bool valid[2];
      i32x4 kb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = tok0 + 16 * h + L16;
        valid[h] = tok >= it.p_lo && tok < it.p_hi;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) mw[h][g] = R.m[h][g];  // (invalid tokens: masked below)
        uint32_t kr[4];
        nib_bytes(R.r[h].x, kr[0], kr[1]);
        nib_bytes(R.r[h].y, kr[2], kr[3]);
        kb[h] = i32x4{(int)kr[0], (int)kr[1], (int)kr[2], (int)kr[3]};
      }
      // the block's two 16-token halves are independent chains sharing each group's digits; the
      // RoPE-key group first (its code bytes come from the lane's own words)
      f32x4 acc[2];
      {
        i32x4 x[2];
        qk_group2(qa[8], kb, x);
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] = bf16f(mw[h][8] & 0xFFFFu) * to_f32x4(x[h]);
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        i32x4 b[2], x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          b[h] = __builtin_bit_cast(i32x4, lds_load<u32x4>(vb + (16 * h + L16) * kVS + 16 * qk_unit<BITS_C>(g, G)));
        qk_group2(qa[g], b, x);
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] += bf16f(mw[h][g] & 0xFFFFu) * to_f32x4(x[h]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f16x8 zlo;
#pragma unroll
        for (int g = 0; g < 8; ++g) zlo[g] = (f16)bf16f(mw[h][g] >> 16);
        const f16 z8 = (f16)bf16f(mw[h][8] >> 16);
        const f16x8 zf = G < 2 ? zlo : f16x8{z8, 0, 0, 0, 0, 0, 0, 0};
        // an invalid token's score is -inf whatever its (possibly unwritten) metadata held
        const f32x4 sc = mfma32k_acc(qz, zf, acc[h] * hs);
        const float ninf = -__builtin_inff();
        S[h] = valid[h] ? sc : f32x4{ninf, ninf, ninf, ninf};
      }
      // online softmax: a head's running max is refreshed only when one of its scores exceeds it
      // by more than kRescale
      bool need = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) need |= (S[0][i] > m_thr[i]) | (S[1][i] > m_thr[i]);
      const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
      if (any) {
        f32x4 alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float m_new = fmaxf(m_run[i], row16_max(fmaxf(S[0][i], S[1][i])));
          alpha[i] = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
          m_run[i] = m_new;
          m_thr[i] = m_new + kRescale;
          m_sub[i] = m_new == -__builtin_inff() ? 0.f : m_new;
          l_part[i] *= alpha[i];
        }
        if (L16 == 0) *reinterpret_cast<f32x4*>(&B.alpha[4 * G]) = alpha;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f16x4 pz;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(S[h][i] - m_sub[i]);
          l_part[i] += e;
          pz[i] = (f16)e;
        }
        *reinterpret_cast<f16x4*>(&B.P[16 * h + L16][4 * G]) = pz;
      }
      // PV scales (normalised) and zeros of groups 2G, 2G + 1 of the lane's two tokens
      // (groups 2 G + q picked by selects: an index that varies across lanes would put mw in
      // scratch memory)
      uint32_t mq[2][2];
      float sg[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t v = mw[h][q];
          asm volatile("" : "+v"(v));  // (keeps the selects from being folded back into an index)
          v = G == 1 ? mw[h][2 + q] : v;
          v = G == 2 ? mw[h][4 + q] : v;
          v = G == 3 ? mw[h][6 + q] : v;
          v = valid[h] ? v : 0u;  // an invalid token gets PV scale and zero 0
          mq[h][q] = v;
          sg[h][q] = bf16f(v & 0xFFFFu);
        }
      int ebit = 0;
      {
        const float smax = fmaxf(fmaxf(sg[0][0], sg[0][1]), fmaxf(sg[1][0], sg[1][1]));
        if (__builtin_amdgcn_ballot_w64(smax >= pv_hi) != 0) {  // rare: raise the exponent
          float m = smax;  // (some lane holds a scale >= pv_hi >= 2^-126: the maximum is a normal number)
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
          const int bits = __builtin_amdgcn_readfirstlane(__float_as_int(m));
          pv_e = min(max(((bits >> 23) & 0xFF) - 127 - 5, -100), 120);
          pv_inv = __builtin_ldexpf(1.f, -pv_e);
          pv_hi = __builtin_ldexpf(1.f, pv_e + 6);
          ebit = 2;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          B.SV[2 * G + q][16 * h + L16] = (f16)(sg[h][q] * pv_inv);
          B.Z[2 * G + q][16 * h + L16] = (f16)bf16f(mq[h][q] >> 16);
        }
      if (lane == 0) {
        B.resc = (any ? 1 : 0) | ebit;
        if (ebit) B.pv_exp = pv_e;
      }
      signal(fl + 0, t, lane);
    };
    if (nb > 0) {
      QRegs R0, R1;  // blocks t, t + 1 (each call issues the same loads, block clamped)
      qload(0, R0);
      qload(1, R1);
      for (int t = 0; t < nb; t += 2) {
        qblock(t, R0);
        qload(t + 2, R0);
        if (t + 1 < nb) qblock(t + 1, R1);
        qload(t + 3, R1);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no loads left in flight at exit
    }
    if (lane == 0 && give_ups) atomicAdd(p.plan_hdr + kHdrGiveUps, give_ups);
    if (lane == 0 && bad_pages) atomicAdd(p.plan_hdr + kHdrBadPages, bad_pages);
    merge_qk(s_tiles.mg, m_run, l_part, pr, G, L16);
  } else {
    // ================================ PV wave of pair pr ================================
    __syncthreads();  // (matches the QK waves' barrier after reading the prologue area)
    struct URegs {
      uint4 c[NLD];
    };
    // the block's content rows are contiguous: 16-byte load i of lane l covers bytes 1024 i + 16 l
    auto uload = [&](int t, URegs& R) {
      int uncounted = 0;  // (the QK wave counts the same pages)
      const uint8_t* base = page_ptr(t, uncounted);
      const int half = (pr + kPairs * min(t, nb - 1)) & 1;
      const uint4* src = reinterpret_cast<const uint4*>(base + half * kPB * CB);
#pragma unroll
      for (int i = 0; i < NLD; ++i) R.c[i] = src[64 * i + lane];
    };
    // code bytes of block t into buffer t % 2 (whole 16-byte units, consecutive lanes consecutive units)
    auto unpack = [&](int t, const URegs& R) {
      uint8_t* vt = &s_tiles.pk[pr][t & 1].V[0][0];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const uint4 v = R.c[i];
        if (BITS_C == 4) {  // 16 bytes = channels 32 c .. 32 c + 31 of token 4 i + l / 16, c = l % 16
          const int row = 4 * i + (lane >> 4), c = lane & 15;
          uint32_t o[8];
          nib_bytes(v.x, o[0], o[1]);
          nib_bytes(v.y, o[2], o[3]);
          nib_bytes(v.z, o[4], o[5]);
          nib_bytes(v.w, o[6], o[7]);
          *reinterpret_cast<uint4*>(vt + row * kVS + 16 * c) = make_uint4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<uint4*>(vt + row * kVS + 16 * (16 + c)) = make_uint4(o[4], o[5], o[6], o[7]);
        } else {  // 16 bytes = group c (64 channels) of token 8 i + l / 8, c = l % 8
          const int row = 8 * i + (lane >> 3), c = lane & 7;
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t x = wd[d];
            *reinterpret_cast<uint4*>(vt + row * kVS + 16 * (8 * d + c)) =
                make_uint4(x & 0x03030303u, (x >> 2) & 0x03030303u, (x >> 4) & 0x03030303u, (x >> 6) & 0x03030303u);
          }
        }
      }
    };
    f32x4 O[32];  // unit u: rows = its bytes 4 G .. 4 G + 3, column head L16
#pragma unroll
    for (int u = 0; u < 32; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oz = {0.f, 0.f, 0.f, 0.f};  // rows z index 4 G + i
    int cur_e = 0;
    auto pv_block = [&](int t) {
      PkBuf& B = s_tiles.pk[pr][t & 1];
      give_ups += wait_at_least(fl + 0, t, spin);  // block t scored
      const lds_ptr<uint8_t> vb = lds_opaque(&B.V[0][0]);
      const lds_ptr<f16> pp = lds_opaque(&B.P[0][0]);
      // B operand base: tokens 8 G .. 8 G + 7 of head L16 (two 4-token transposed reads)
      const f16x8 pv = cat8(lds_tr4(pp + (8 * G + (L16 >> 2)) * kPkP + 4 * (L16 & 3)),
                            lds_tr4(pp + (8 * G + 4 + (L16 >> 2)) * kPkP + 4 * (L16 & 3)));
      const int resc = __builtin_amdgcn_readfirstlane(B.resc);
      if (resc) {
        const float a = (resc & 1) ? B.alpha[L16] : 1.f;
        float ae = a;
        if (resc & 2) {  // the PV scales now carry 2^-pv_exp: bring the sums to that scale
          const int ne = __builtin_amdgcn_readfirstlane(B.pv_exp);
          ae = a * __builtin_ldexpf(1.f, cur_e - ne);
          cur_e = ne;
        }
#pragma unroll
        for (int u = 0; u < 32; ++u) O[u] *= ae;
        oz *= a;
      }
      const f16x8 zA = L16 < 8 ? *reinterpret_cast<const f16x8*>(&B.Z[L16 & 7][8 * G]) : f16x8{};
      oz = mfma32k_acc(zA, pv, oz);
      // code column of unit u: rows 8 G .. 8 G + 7 (tokens), 16 columns; lane L16 gets column L16.
      // Software pipeline: the four code columns and the PV scales of group g + 1 are requested
      // before group g multiplies (the scheduling fences keep the requests in place).
      const lds_ptr<uint8_t> colp = vb + (8 * G + (L16 >> 1)) * kVS + 8 * (L16 & 1);
      u32x2 raw[2][4];
      f16x8 svr[2];
      auto request = [&](int g) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          raw[g & 1][q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                                       reinterpret_cast<lds_ptr<i32x2>>(colp + 16 * qk_unit<BITS_C>(g, q))));
        svr[g & 1] = *reinterpret_cast<const f16x8*>(&B.SV[g][8 * G]);
      };
      request(0);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        if (g + 1 < 8) request(g + 1);
        __builtin_amdgcn_sched_barrier(0);
        const f16x8 bop = pv * svr[g & 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = qk_unit<BITS_C>(g, q);
          O[u] = mfma32k_acc(codes_to_f16(raw[g & 1][q]), bop, O[u]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if (nb > 0) {
      // one block of content words in registers: block t + 3 is requested after block t + 2 is
      // unpacked, one iteration before it is needed
      URegs R;
      uload(0, R);
      unpack(0, R);
      signal(fl + 1, 0, lane);
      uload(1, R);
      unpack(1, R);  // (nb == 1: the clamped copy of block 0 goes to buffer 1, never read)
      signal(fl + 1, 1, lane);
      uload(2, R);
      for (int t = 0; t < nb; ++t) {
        pv_block(t);
        if (t + 2 < nb) {
          unpack(t + 2, R);
          signal(fl + 1, t + 2, lane);
          uload(t + 3, R);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no loads left in flight at exit
    }
    if (lane == 0 && give_ups) atomicAdd(p.plan_hdr + kHdrGiveUps, give_ups);
    const int64_t orow = (int64_t)it.item * p.heads + it.head0 + L16;
    merge_pv(p, s_tiles.mg, O, oz, cur_e + 24, pr, lane, G, L16, orow, false, 0,
             [&](f32x4(&Of)[32], const float(&)[8], float) {
      float* dst = p.ws_o + orow * kDc;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const f32x4 v = Of[u];
        const int base = pk_unit_base<BITS_C>(u);
        if (BITS_C == 4) {
          // lanes G and G ^ 1 hold channels base + 8 (G >> 1) + {0 2 4 6 | 1 3 5 7}: each takes two
          // values from the other, so lane G even holds 0..3 and lane G odd 4..7 of those 8
          const bool odd = G & 1;
          const float rx = __shfl_xor(odd ? v[0] : v[2], 16, 64);
          const float ry = __shfl_xor(odd ? v[1] : v[3], 16, 64);
          const f32x4 r = odd ? f32x4{rx, v[2], ry, v[3]} : f32x4{v[0], rx, v[1], ry};
          *reinterpret_cast<f32x4*>(dst + base + 8 * (G >> 1) + 4 * (G & 1)) = r;
        } else {
          // register i of lane G holds channel base + 4 i + G
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[base + 4 * i + G] = v[i];
        }
      }
    });
  }
}

template <int BITS_C>
__global__ __launch_bounds__(kThreads) void decode16_kernel(DecodeParams p) {
  using GE = Geo<BITS_C>;
  __shared__ Tiles16 s_tiles;
  __shared__ int s_flag[kPairs][4];  // [pair][published block, released block, -, -]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = w & (kPairs - 1);  // pair
  const int G = lane >> 4;
  const int L16 = lane & 15;

  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int hg = kx % p.head_groups;
  const int item = xcd + 8 * (kx / p.head_groups);
  if (item >= min(p.plan_hdr[kHdrItems], p.max_items)) return;
  const int4 itm = reinterpret_cast<const int4*>(p.items)[item];
  const int b = itm.x;
  const bool packed = itm.w == 0;

  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  const int p_lo = p.n_sink, p_hi = N - p.n_recent;
  const int first_page = p_lo / kPageTokens;
  const int n_pp = p_hi > p_lo ? (p_hi - 1) / kPageTokens - first_page + 1 : 0;
  // n_blocks: the pair's 16-token blocks.  A bf16 item holds entries [jb, nb) of the sequence's
  // bf16 token list (sink tokens, then the recent window from rstart on), in virtual pages of 64.
  int n_blocks, page0 = 0, ns = 0, nb = 0, rstart = 0, jb = 0;
  if (!packed) {
    ns = min(p.n_sink, N);
    rstart = max(p.n_sink, N - p.n_recent);
    jb = max(0, itm.y);
    nb = min(bf16_token_count(N, p.n_sink, p.n_recent), jb + max(0, itm.z));
    n_blocks = nb > jb ? (nb - jb + kPageTokens - 1) / kPageTokens : 0;
  } else {
    page0 = itm.y;
    n_blocks = min(min(itm.z, first_page + n_pp - page0), p.max_pages - page0);
    if (n_blocks <= 0) return;
  }
  if (packed && p.num_pages <= 0) return;

  const int head0 = hg * 16;
  const float c_log2 = p.scale_log2e;
  const int last = n_blocks - 1;

  if (tid < kPairs * 4) (&s_flag[0][0])[tid] = -1;
  // LDS addressing: one base pointer per LDS object plus a byte offset (the pair's two buffers
  // are kPT apart; block t uses buffer t % 2)
  const lds_ptr<uint8_t> tb = (lds_ptr<uint8_t>)&s_tiles;
  lds_vint* const fl = (lds_vint*)&s_flag[pr][0];
  constexpr int kPT = (int)sizeof(PairTiles);
  constexpr int oP = (int)offsetof(PairTiles, P), oZ = (int)offsetof(PairTiles, Z);
  constexpr int oSV = (int)offsetof(PairTiles, SV), oA = (int)offsetof(PairTiles, alpha);
  constexpr int oR = (int)offsetof(PairTiles, resc);
  const int pb0 = pr * 2 * kPT;  // the pair's first buffer
  const int rsel = 4 * G + (L16 >> 2), csel = 4 * (L16 & 3);
  const int o_vtr = pb0 + 2 * (rsel * kSV + csel);       // V^T operand, + 32 per 16 channel positions
  const int o_vwr = pb0 + 2 * (L16 * kSV + 16 * G);      // V row slice, + 128 per group
  const int o_ptr = pb0 + oP + 2 * (rsel * kPS + csel);  // P^T operand
  const int o_pwr = pb0 + oP + 2 * (L16 * kPS + 4 * G);
  const int o_ztr = pb0 + oZ + 2 * (rsel * kPS + csel);
  const int o_zwr = pb0 + oZ + 2 * (L16 * kPS);
  const int o_svr = pb0 + oSV + 8 * G;                   // + 32 per group
  const int o_svw = pb0 + oSV + 2 * L16;
  const int o_al = pb0 + oA;
  const int o_rs = pb0 + oR;
  __syncthreads();  // flags initialised
  if (packed) {
    const ItemCtx ctx{item, b, slot, p_lo, p_hi, page0, n_blocks, head0};
    packed_item<BITS_C>(p, s_tiles, s_flag, ctx);
    return;
  }

  auto& mg = s_tiles.mg;
  const int spin = p.spin_limit;
  int give_ups = 0;  // (uniform across the wave)
  if (w < kPairs) {
    // ============================== QK wave of pair pr ==============================
    const int row = 16 * pr + L16;  // the lane's token row within a page
    // queries: A operand (lane: head head0 + L16; K step (g, h): channels 64g + 16G + 8h .. +7)
    f16x8 qreg[18];
    f16x8 qz;
    auto load_queries = [&]() {
      float qs[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) qs[g] = 0.f;
      const uint16_t* qh = p.q + ((int64_t)b * p.heads + head0 + L16) * kD;
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 raw = *reinterpret_cast<const uint4*>(qh + 64 * g + 16 * G + 8 * h);
          const uint4 hv = g < 8 ? bf16_chunk_to_f16<BITS_C>(raw) : bf16_chunk_to_f16<4>(raw);
          qreg[2 * g + h] = __builtin_bit_cast(f16x8, hv);
          float sum = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) sum += (float)qreg[2 * g + h][j];
          qs[g] += sum;
        }
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        qs[g] += __shfl_xor(qs[g], 16, 64);
        qs[g] += __shfl_xor(qs[g], 32, 64);
        qs[g] *= c_log2;
      }
      // zero-term step, k = 8 G + j: G0 hi(qsum_j), G1 lo(qsum_j) against z_j; G2 / G3 hi / lo of
      // qsum_8 in slot j = 0 against z_8 (the other slots meet zeros)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = G < 2 ? qs[j] : (j == 0 ? qs[8] : 0.f);
        const f16 hi = (f16)x;
        const f16 lo = (f16)(x - (float)hi);
        qz[j] = (G & 1) ? lo : hi;
      }
    };
    if (G == 0) {  // Z columns 8 .. 15 of both buffers
      *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_zwr + 16)) = f16x8{};
      *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_zwr + kPT + 16)) = f16x8{};
    }

    float m_run[4], l_part[4];  // heads 4G + i (the lane's S rows)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[i] = -__builtin_inff();
      l_part[i] = 0.f;
    }
    auto needs_refresh = [&](f32x4 S) {
      bool need = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) need |= S[i] > m_run[i] + kRescale;
      return __builtin_amdgcn_ballot_w64(need) != 0;
    };
    // refresh the running maxima; the PV wave gets the per-head factor with the block
    auto refresh = [&](f32x4 S, int so) {
      f32x4 alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m_new = fmaxf(m_run[i], row16_max(S[i]));
        alpha[i] = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
        m_run[i] = m_new;
        l_part[i] *= alpha[i];
      }
      if (L16 == 0) *reinterpret_cast<lds_ptr<f32x4>>(tb + (o_al + so + 16 * G)) = alpha;
    };
    // softmax of block t with the current running maxima, probabilities to the P tile, publish
    auto publish = [&](f32x4 S, int t, int resc, int so) {
      f16x4 pz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mu = m_run[i] == -__builtin_inff() ? 0.f : m_run[i];
        const float e = __builtin_amdgcn_exp2f(S[i] - mu);
        l_part[i] += e;
        pz[i] = (f16)e;
      }
      *reinterpret_cast<lds_ptr<f16x4>>(tb + (o_pwr + so)) = pz;
      if (lane == 0) *reinterpret_cast<lds_ptr<int>>(tb + (o_rs + so)) = resc;
      signal(fl + 0, t, lane);
    };
    // the QK of one block from the rows' fp16 K steps kf16(g, h), their scales and zeros in mw
    // (bf16 s | z << 16: 1 and 0 for valid tokens, 0 for masked ones); writes the V, Z and SV
    // tiles, returns S (rows heads 4G + i, column token L16)
    auto block_qk = [&](auto&& kf16, const uint32_t* mw, bool valid, int so) -> f32x4 {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kGroups; ++i) {  // groups 8 (RoPE key), 0, 1, .., 7: the RoPE-key product first
        const int g = i == 0 ? kGroups - 1 : i - 1;
        const f16x8 k0 = kf16(g, 0), k1 = kf16(g, 1);
        f32x4 c = mfma32k(qreg[2 * g], k0, f32x4{0.f, 0.f, 0.f, 0.f});
        c = mfma32k(qreg[2 * g + 1], k1, c);
        s += bf16f(mw[g] & 0xFFFFu) * c;
        if (g < 8) {
          *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_vwr + so + 128 * g)) = k0;
          *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_vwr + so + 128 * g + 16)) = k1;
        }
      }
      // The token's zeros in fp16 (every lane holds its token's nine), the zero-term operand from
      // them (z_0 .. z_7 for G < 2, z_8 and zeros for G >= 2), and the Z and SV tile entries: lanes
      // G = 0 write the token's Z row, lane G writes the PV scales of groups 2G, 2G + 1.
      f16x8 zlo;
#pragma unroll
      for (int g = 0; g < 8; ++g) zlo[g] = (f16)bf16f(mw[g] >> 16);
      const f16 z8 = (f16)bf16f(mw[8] >> 16);
      const f16x8 zf = G < 2 ? zlo : f16x8{z8, 0, 0, 0, 0, 0, 0, 0};
      {
        const uint32_t a0 = (G & 1) ? mw[2] : mw[0], b0 = (G & 1) ? mw[6] : mw[4];
        const uint32_t a1 = (G & 1) ? mw[3] : mw[1], b1 = (G & 1) ? mw[7] : mw[5];
        const uint32_t m0 = (G & 2) ? b0 : a0, m1 = (G & 2) ? b1 : a1;
        const float s0 = bf16f(m0 & 0xFFFFu), s1 = bf16f(m1 & 0xFFFFu);
        *reinterpret_cast<lds_ptr<f16>>(tb + (o_svw + so + 64 * G)) = (f16)s0;
        *reinterpret_cast<lds_ptr<f16>>(tb + (o_svw + so + 64 * G + 32)) = (f16)s1;
        if (G == 0) {
          *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_zwr + so)) = zlo;
          *reinterpret_cast<lds_ptr<f16>>(tb + (o_zwr + so + 16)) = z8;
        }
      }
      return mfma32k(qz, zf, s * c_log2) + (valid ? 0.f : -__builtin_inff());
    };

    {
      // bf16 tokens in virtual pages of 64, the pair's rows 16 pr .. 16 pr + 15 of each.  With
      // several query tokens, this workgroup's query sees the first n_vis tokens (the ones it does
      // not see are all in the recent window, so only bf16 items mask them).
      const int n_vis = N - (p.q_len - 1 - head0 / p.heads_per_query);
      load_queries();
      for (int t = 0; t < n_blocks; ++t) {
        const int j = jb + t * kPageTokens + row;
        const bool valid = j < nb && (j < ns ? j : rstart + (j - ns)) < n_vis;
        // every lane loads (rows past the list or not seen read the slot's first recent row and are
        // dropped), so that the block's 18 loads are issued together
        const bool in = j < nb;
        const uint16_t* src = p.recent + (int64_t)slot * p.n_recent * kD;
        if (in && j < ns) src = p.sink + ((int64_t)slot * p.n_sink + j) * kD;
        else if (in) src = p.recent + ((int64_t)slot * p.n_recent + (rstart + (j - ns)) % p.n_recent) * kD;
        uint4 raw[2 * kGroups];
#pragma unroll
        for (int k = 0; k < 2 * kGroups; ++k) raw[k] = *reinterpret_cast<const uint4*>(src + 64 * (k >> 1) + 16 * G + 8 * (k & 1));
        // scale 1 (bf16 0x3F80) and zero 0 for valid tokens
        uint32_t mw[kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) mw[g] = valid ? 0x3F80u : 0u;
        auto kf16 = [&](int g, int h) -> f16x8 {
          const uint4 r = valid ? raw[2 * g + h] : make_uint4(0, 0, 0, 0);
          return __builtin_bit_cast(f16x8, g < 8 ? bf16_chunk_to_f16<BITS_C>(r) : bf16_chunk_to_f16<4>(r));
        };
        const int so = (t & 1) * kPT;
        give_ups += wait_at_least(fl + 1, t - 2, spin);  // buffer t % 2 is free
        const f32x4 S = block_qk(kf16, mw, valid, so);
        const bool resc = needs_refresh(S);
        if (resc) refresh(S, so);
        publish(S, t, resc ? 1 : 0, so);
      }
    }
    if (lane == 0 && give_ups) atomicAdd(p.plan_hdr + kHdrGiveUps, give_ups);
    merge_qk(mg, m_run, l_part, pr, G, L16);
  } else {
    // ============================== PV wave of pair pr ==============================
    f32x4 O[32];  // column head L16, rows channel positions 16 cb + 4G + i
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) O[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oz = {0.f, 0.f, 0.f, 0.f};  // rows z index 4G + i
    for (int t = 0; t < n_blocks; ++t) {
      give_ups += wait_at_least(fl + 0, t, spin);  // block t published
      // block t's operands into registers (k = tokens 4G .. 4G + 3), then release its buffer
      const int so = (t & 1) * kPT;
      const f16x4 pb = lds_tr4((lds_ptr<f16>)(tb + (o_ptr + so)));  // B: head L16
      const f16x4 za = lds_tr4((lds_ptr<f16>)(tb + (o_ztr + so)));  // A: z index L16
      f16x4 sv[8], va[32];
#pragma unroll
      for (int g = 0; g < 8; ++g) sv[g] = lds_load<f16x4>(tb + (o_svr + so + 32 * g));
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) va[cb] = lds_tr4((lds_ptr<f16>)(tb + (o_vtr + so + 32 * cb)));
      const int resc = __builtin_amdgcn_readfirstlane(lds_load<int>(tb + (o_rs + so)));
      const float alpha = lds_load<float>(tb + (o_al + so + 4 * L16));
      signal(fl + 1, t, lane);
      if (resc) {
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) O[cb] *= alpha;
        oz *= alpha;
      }
      oz = mfma16k(za, pb, oz);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const f16x4 bop = pb * sv[g];
#pragma unroll
        for (int c = 0; c < 4; ++c) O[4 * g + c] = mfma16k(va[4 * g + c], bop, O[4 * g + c]);
      }
    }
    if (lane == 0 && give_ups) atomicAdd(p.plan_hdr + kHdrGiveUps, give_ups);
    const int64_t orow = (int64_t)item * p.heads + head0 + L16;
    // a sequence decoded by this item alone gets its final outputs here (workgroup-uniform)
    const bool direct = decoded_in_one_item(p, b);
    if (direct && pr == 0 && lane == 0) atomicAdd(p.plan_hdr + kHdrDirect, 1);  // (PV waves run this)
    const int64_t out_row = (int64_t)b * p.heads + head0 + L16;
    merge_pv(p, mg, O, oz, 0, pr, lane, G, L16, orow, direct, out_row,
             [&](f32x4(&Of)[32], const float(&zs)[8], float inv) {
      float* dst = p.ws_o + orow * kDc;
      uint16_t* od = p.out + out_row * kDc;
      // Lanes G and G ^ 1 (lane ^ 16) hold the 8 channels 16 cb + 8 (G >> 1) + 0..7 between them,
      // in the unpacking order; each takes two values from the other so that lane G even holds
      // channels 0..3 and lane G odd channels 4..7, written as one 16-byte store.
      const bool odd = G & 1;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        const f32x4 v = Of[cb];
        f32x4 r;
        if (BITS_C == 4) {  // even lane: channels 0 2 4 6, odd lane: 1 3 5 7
          const float rx = __shfl_xor(odd ? v[0] : v[2], 16, 64);
          const float ry = __shfl_xor(odd ? v[1] : v[3], 16, 64);
          r = odd ? f32x4{rx, v[2], ry, v[3]} : f32x4{v[0], rx, v[1], ry};
        } else {            // even lane: channels 0 4 1 5, odd lane: 2 6 3 7
          const float rx = __shfl_xor(odd ? v[0] : v[1], 16, 64);
          const float ry = __shfl_xor(odd ? v[2] : v[3], 16, 64);
          r = odd ? f32x4{rx, ry, v[1], v[3]} : f32x4{v[0], v[2], rx, ry};
        }
        const int c0 = 16 * cb + 8 * (G >> 1) + 4 * (G & 1);  // channels c0 .. c0 + 3, group cb / 4
        if (direct) store_bf16x4(od + c0, (r + zs[cb >> 2]) * inv);
        else *reinterpret_cast<f32x4*>(dst + c0) = r;
      }
    });
  }
}

template <int BITS_C>
hipError_t launch16(const DecodeParams& p, hipStream_t stream) {
  const int64_t blocks = ((int64_t)p.max_items + 7) / 8 * 8 * p.head_groups;
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(decode16_kernel<BITS_C>), dim3((unsigned)blocks),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_decode16(const DecodeParams& p, int bits_c, hipStream_t stream) {
  if (bits_c == 4) return launch16<4>(p, stream);
  if (bits_c == 2) return launch16<2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
