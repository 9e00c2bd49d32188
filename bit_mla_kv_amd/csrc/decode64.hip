// Split-KV low-bit MLA decode for groups of 64 query heads on gfx950 (CDNA4).
//
// Same computation as decode.hip (QuantMLA pages: ai.info summary, "Key
// Contributions", item 4; onedev.kr review, "How it is used"): one global
// softmax over all valid tokens, sink / recent tokens from bf16, all others
// from their packed copies, output aggregated over the content latent.
//
// One workgroup of 8 waves per (sequence, split, 64-head group), one QK wave
// and one PV wave on each SIMD, so that the MFMA and VALU work of a step is
// spread evenly over the four SIMDs:
//  - QK waves 0..3 hold the queries of 16 heads each and score one 32-token
//    tile per step with MFMA 16x16x32 f16 (queries as the A operand, so each
//    lane owns one token of a 16-token block and applies that token's fp32
//    group scales as scalars).  The zero terms of all nine groups go through
//    one more MFMA against the tile's zero columns with qsum split into fp16
//    hi + lo; it also adds each token's score mask (0, or -inf for a token
//    outside the item) and takes the group-scaled sum as its accumulator, so
//    the score leaves it complete.  Online softmax in the log2 domain with a
//    lazily refreshed running max; probabilities are published to LDS as fp16
//    [token][head], token rows permuted for the LDS banks (p_row below).
//    The same waves also load the packed bytes of the tile three steps ahead
//    into registers and unpack the next tile into an fp16 tile of exact codes
//    (nibbles / crumbs become fp8 bytes whose e4m3 value is code * 2^-9,
//    converted with a 2^9 scale) plus per-token scales, zeros and masks; they
//    take a quarter of the content codes, the RoPE-key codes and the metadata;
//  - PV waves 4..7 hold the output of content groups 2v, 2v+1 (v = w - 4) for
//    all 64 heads and accumulate p * s_g times the exact codes (MFMA 32x32x16
//    f16, both operands read with the LDS transpose load) plus the zero-term
//    sums sum_t p_t z_g,t, whose ones column also gives each head's sum of
//    probabilities.  They load and unpack the rest of the content codes, so
//    both roles of a SIMD share the unpacking work (the split that measured
//    fastest: the QK waves carry the softmax and the metadata).
// Tiles flow through a three-slot LDS ring, one workgroup barrier per tile: in
// step k the QK waves score tile k (MFMAs first, then the softmax and their
// share of the unpacking of tile k + 1) and the PV waves accumulate tile k - 1
// (their unpacking first, then the MFMAs), so that each role's VALU work meets
// the other's MFMAs on the shared SIMD.  The token order of each MFMA's k slots
// is chosen so that the LDS accesses of a step fall on distinct banks.
// Partials are left unnormalised with their running max and sum; the combine
// kernel adds the zero terms and merges splits.  A sequence decoded in one item
// gets its final outputs and lse here instead.
#include <algorithm>
#include <type_traits>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kT = 32;            // tokens per tile (half a page)
constexpr int kHW = 64;           // query heads per workgroup
constexpr int kThreads = 512;     // 4 QK + unpack waves, 4 PV waves
constexpr int kSlots = 3;         // tile ring
constexpr int kS = 592;           // tile row stride (halves): 576 codes + 16 zero-term columns
constexpr int kZ = 576;           // zero-term columns: z_0..z_7, z_8, the score mask, 1, five zeros
constexpr int kPT = 68;           // probability row stride (halves); row p_row(t) holds token t
constexpr float kRescale = 8.0f;  // lazy max refresh threshold, log2 units

template <int BITS_C>
struct Geo {
  static constexpr int CB = kDc * BITS_C / 8;                              // content bytes per token
  static constexpr int PB = kPageTokens * (CB + kDr / 2 + 4 * kGroups);   // page bytes
  static constexpr int ROPE0 = kPageTokens * CB;                           // RoPE block of a page
  static constexpr int META0 = kPageTokens * (CB + kDr / 2);               // metadata block of a page
  static constexpr int CDW = kT * CB / 4;      // content dwords of a tile
  static constexpr int DPR = CB / 4;           // content dwords per token
  static constexpr int CPT = CDW / 256;        // content dwords per thread index (QK and PV threads share them)
  static constexpr int CQ = CPT / 4;           // content dwords a QK thread unpacks; a PV thread takes the rest
  static constexpr int RPT = kT * kDr / 8 / 256;  // RoPE dwords per unpack thread (1)
  static_assert(CDW % 256 == 0 && RPT == 1, "unpack split assumes these sizes");
};

// packed bytes of one tile held by an unpack thread: content, RoPE, and the metadata words of
// (token t % 32, group t / 32) and (token t % 32, group 8) for thread t
template <int BITS_C>
struct TileRegs {
  uint32_t c[Geo<BITS_C>::CQ];
  uint32_t r;
  uint32_t m[2];
};
// the content dwords of a tile a PV thread loads and unpacks
template <int BITS_C>
struct PVRegs {
  uint32_t c[Geo<BITS_C>::CPT - Geo<BITS_C>::CQ];
};

// Page id of page_idx of the slot's block table, read through the constant address space (scalar
// loads); an index or id outside the table or the pool reads page 0 (wrong values, no fault) and
// is counted in *bad (uniform across the wave).
typedef __attribute__((address_space(4))) const int32_t cint;
__device__ __forceinline__ int64_t page_of(const DecodeParams& p, cint* bt, int page_idx, int* bad) {
  int64_t pg = (page_idx < p.max_pages) ? (int64_t)bt[min(page_idx, p.max_pages - 1)] : -1;
  if (pg < 0 || pg >= p.num_pages) {
    pg = 0;
    ++*bad;
  }
  return pg;
}

// content dwords u = ft + 256 i (i in [I0, I0 + n)) of a tile: unpacked into the tile rows
template <int BITS_C, int I0, int NI>
__device__ __forceinline__ void unpack_content(f16* tile, int ft, const uint32_t (&c)[NI]) {
  using GE = Geo<BITS_C>;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int u = ft + 256 * (I0 + i);
    const int r = u / GE::DPR, d = u % GE::DPR;
    f16* dst = &tile[r * kS];
    if (BITS_C == 4) {
      *reinterpret_cast<uint4*>(dst + 8 * d) = unpack4(c[i]);
    } else {
      uint4 x0, x1;
      unpack2(c[i], x0, x1);
      *reinterpret_cast<uint4*>(dst + 16 * d) = x0;
      *reinterpret_cast<uint4*>(dst + 16 * d + 8) = x1;
    }
  }
}

template <int BITS_C>
struct __align__(16) Smem64 {
  f16 tile[kSlots][kT * kS];       // exact codes of a tile's tokens + zero-term columns
  f16 probT[2][kT][kPT];           // fp16 probabilities [token][head] of steps k (QK) and k - 1 (PV)
  float sq[kSlots][kGroups][kT];   // s_g * scale * log2 e at sq_pos(token); 0 for masked tokens
  f16 svh[kSlots][8][kT];          // PV group scale s_g * 2^-E_g (fp16) at pv_pos(token); 0 for masked tokens
  float alpha[2][kHW];             // per-head rescale factor for the PV accumulators
  int resc[2][4];                  // per-QK-wave flags: bit 0 some head was rescaled, bit 1 the wave's
                                   // groups changed their PV scale exponent
  int pve[kSlots][8];              // PV scale exponent E_g of a tile: svh holds fp16(s_g * 2^-E_g)
};

// Per-token QK constants sit so that one 8-byte read gives a lane the values of its token in
// both 16-token blocks: token r at 2 * (r % 16) + r / 16.
__device__ __forceinline__ int sq_pos(int r) { return 2 * (r & 15) + (r >> 4); }

// LDS bank placement of the probabilities and the PV operand reads.  The token order of an MFMA's
// k slots is free, so it is chosen for the banks (as measured on gfx950: 16-byte reads go in four
// passes of 16 lanes over 64 banks, 8-byte and transposed reads in two passes of 32 lanes over 64
// banks, 8-byte writes in four passes of 16 lanes over 32 banks).  Token t = 16h + 8a + 4c + 2d + e
// (one bit each):
//  - its probabilities sit in row p_row(t) = 16h + 8d + 4e + 2(c^h) + a: with a row stride of 34
//    dwords the QK wave's two 8-byte writes (tokens L16 and 16 + L16) cover all 32 banks per pass;
//  - a PV read pass takes the four tokens of set x (x = ks + 2 rd + 4 half; a = x & 1,
//    c^h = (x >> 1) & 1, e = x >> 2, slot j = d + 2h): their tile rows (stride 296 dwords) and
//    probability rows fall on four distinct 16-bank windows each;
//  - the zero-term reads take the eight tokens of sets x and x + 4 per pass, distinct 8-bank
//    windows in both buffers;
//  - its PV scale sits at pv_pos(t), so that the eight scales of (ks, half) are one 16-byte read in
//    register order (rd = 0 then rd = 1).
__device__ __forceinline__ int p_row(int t) {
  const int h = (t >> 4) & 1, a = (t >> 3) & 1, c = (t >> 2) & 1, d = (t >> 1) & 1, e = t & 1;
  return 16 * h + 8 * d + 4 * e + 2 * (c ^ h) + a;
}
__device__ __forceinline__ int pv_token(int x, int j) {
  const int d = j & 1, h = j >> 1;
  return 16 * h + 8 * (x & 1) + 4 * (((x >> 1) & 1) ^ h) + 2 * d + (x >> 2);
}
__device__ __forceinline__ int pv_pos(int t) {
  const int h = (t >> 4) & 1, a = (t >> 3) & 1, c = (t >> 2) & 1, d = (t >> 1) & 1, e = t & 1;
  return 16 * a + 8 * e + 4 * (c ^ h) + 2 * h + d;
}

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// max over the 16 lanes of a row (lanes 16k .. 16k + 15)
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

template <int BITS_C>
__global__ __launch_bounds__(kThreads) void decode64_kernel(DecodeParams p) {
  using GE = Geo<BITS_C>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem64<BITS_C>& sm = *reinterpret_cast<Smem64<BITS_C>*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar: roles branch uniformly
  const int G = lane >> 4;       // 16x16x32 k slice / D row block
  const int L16 = lane & 15;
  const int half = lane >> 5;    // 32x32x16 k half
  const int l32 = lane & 31;

  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int hg = kx % p.head_groups;
  const int item = xcd + 8 * (kx / p.head_groups);
  if (item >= min(p.plan_hdr[kHdrItems], p.max_items)) return;
  const int4 itm = reinterpret_cast<const int4*>(p.items)[item];
  const int b = itm.x;
  const bool packed = itm.w == 0;  // otherwise the item holds the sequence's bf16 tokens

  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  const int p_lo = p.n_sink, p_hi = N - p.n_recent;
  const int first_page = p_lo / kPageTokens;
  const int n_pp = p_hi > p_lo ? (p_hi - 1) / kPageTokens - first_page + 1 : 0;
  // a bf16 item holds entries [jb, nb) of the sequence's bf16 token list (sink tokens, then the
  // recent window from rstart on)
  int n_tiles, page0 = 0, ns = 0, nb = 0, rstart = 0, jb = 0;
  if (!packed) {
    ns = min(p.n_sink, N);
    rstart = max(p.n_sink, N - p.n_recent);
    jb = max(0, itm.y);
    nb = min(bf16_token_count(N, p.n_sink, p.n_recent), jb + max(0, itm.z));
    n_tiles = nb > jb ? (nb - jb + kT - 1) / kT : 0;
  } else {
    page0 = itm.y;
    n_tiles = 2 * min(itm.z, first_page + n_pp - page0);
    if (n_tiles <= 0) return;
  }

  if (packed && p.num_pages <= 0) return;  // packed tokens without a page pool: nothing to read
  // every role runs the same n_steps = n_tiles + 1 steps (one barrier each), rounded up to a
  // multiple of 3 so the unpack waves cycle through their three register buffers in step
  const int n_steps = (n_tiles + 3) / 3 * 3;

  const int head0 = hg * kHW;
  const float c_log2 = p.scale_log2e;
  const int64_t row0 = (int64_t)item * p.heads + head0;  // first workspace row of this workgroup
  // A sequence decoded by this item alone (a bf16 item, no packed chunk) gets its final outputs
  // and lse here, as the combine would compute them from this one partial: the QK waves hand each
  // head's running max and sum, the PV waves the zero-term sums, through the then unused tile
  // slot 0 (one more workgroup barrier, taken by every wave).
  const bool direct = !packed && decoded_in_one_item(p, b);
  const int64_t orow0 = (int64_t)b * p.heads + head0;  // first output row of this workgroup
  float* x_ml = reinterpret_cast<float*>(&sm.tile[0][0]);  // [64 heads][2]: m, l
  float* x_z = x_ml + 2 * kHW;                               // [64 heads][8]: zero-term sums

  // bf16 items: the 16-byte chunks of a tile's rows (32 tokens x 72 chunks) are spread over all
  // 512 threads (chunk tid + 512 e; the fifth, e = 4, exists only for the QK threads), requested at
  // the start of a step and converted into the tile at its end, so their latency hides behind the
  // step's QK / PV work
  constexpr int kBfChunks = kT * (kD / 8);
  static_assert(kBfChunks == 4 * kThreads + 256, "chunk split assumes 2304 chunks a tile");
  constexpr int kBfQK = 5, kBfPV = 4;
  struct BfRegs {
    uint4 x[kBfQK];
  };
  auto bf_load = [&](int t, BfRegs& R, auto per) {
#pragma unroll
    for (int e = 0; e < decltype(per)::value; ++e) {
      const int u = tid + kThreads * e, r = u / (kD / 8), m = u % (kD / 8);
      const int j = jb + t * kT + r;
      R.x[e] = make_uint4(0, 0, 0, 0);
      if (u < kBfChunks && j < nb) {
        const uint16_t* src = j < ns ? p.sink + ((int64_t)slot * p.n_sink + j) * kD
                                     : p.recent + ((int64_t)slot * p.n_recent + (rstart + (j - ns)) % p.n_recent) * kD;
        R.x[e] = *reinterpret_cast<const uint4*>(src + 8 * m);
      }
    }
  };
  auto bf_store = [&](int t, const BfRegs& R, auto per) {
    f16* tile = &sm.tile[t % kSlots][0];
#pragma unroll
    for (int e = 0; e < decltype(per)::value; ++e) {
      const int u = tid + kThreads * e, r = u / (kD / 8), m = u % (kD / 8);
      if (u < kBfChunks)
        *reinterpret_cast<uint4*>(&tile[r * kS + 8 * m]) =
            m < kDc / 8 ? bf16_chunk_to_f16<BITS_C>(R.x[e]) : bf16_chunk_to_f16<4>(R.x[e]);
    }
  };

  if (w < 4) {
    // ====== QK + unpack waves: QK of heads head0 + 16w + L16, unpacking of a quarter of each tile ======
    const int ft = tid;  // 0 .. 255
    cint* bt = (cint*)(uintptr_t)(p.block_table + (int64_t)slot * p.max_pages);
    int bad_pages = 0;
    // packed bytes of tile min(t, n_tiles - 1) (half t % 2 of page page0 + t / 2) into registers;
    // every call issues the same loads, so the compiler's load counting stays exact
    auto load = [&](int t, TileRegs<BITS_C>& R) {
      t = min(t, n_tiles - 1);
      const int hs = t & 1;
      const uint8_t* base = p.pages + page_of(p, bt, page0 + (t >> 1), &bad_pages) * (int64_t)GE::PB;
      const uint32_t* srcC = reinterpret_cast<const uint32_t*>(base + hs * kT * GE::CB);
      const uint32_t* srcR = reinterpret_cast<const uint32_t*>(base + GE::ROPE0 + hs * kT * kDr / 2);
      const uint32_t* srcM = reinterpret_cast<const uint32_t*>(base + GE::META0 + hs * kT * 4 * kGroups);
#pragma unroll
      for (int i = 0; i < GE::CQ; ++i) R.c[i] = srcC[ft + 256 * i];
      R.r = srcR[ft];
      R.m[0] = srcM[(ft & 31) * kGroups + (ft >> 5)];
      R.m[1] = srcM[(ft & 31) * kGroups + 8];
    };
    // PV scale normaliser of a packed item, per group (this thread's group ft / 32: lanes 0..31 of
    // wave w hold group 2w, lanes 32..63 group 2w + 1): the tile gets fp16(s * 2^-pv_e), pv_e raised
    // (never lowered) so that the largest scale seen so far sits in [2^5, 2^6); with probabilities
    // <= 2^8 (lazy max refresh) every PV product p * s * 2^-pv_e stays below 2^14.
    int pv_e = 0, echg = 0;
    float pv_inv = 1.f, pv_hi = 0x1p-126f;  // 2^-pv_e; raise when a scale reaches pv_hi = 2^(pv_e + 6)
    // unpack tile t into ring slot t % 3
    auto fill = [&](int t, const TileRegs<BITS_C>& R) {
      const int sl = t % kSlots;
      f16* tile = &sm.tile[sl][0];
      if (!packed) {  // the rows themselves come through bf_load / bf_store
        if (ft < kT) {
          const int r = ft;
          const bool valid = jb + t * kT + r < nb;
#pragma unroll
          for (int g = 0; g < kGroups; ++g) sm.sq[sl][g][sq_pos(r)] = valid ? c_log2 : 0.f;
#pragma unroll
          for (int g = 0; g < 8; ++g) sm.svh[sl][g][pv_pos(r)] = valid ? (f16)1.f : (f16)0.f;
          *reinterpret_cast<uint4*>(&tile[r * kS + kZ]) = make_uint4(0, 0, 0, 0);
          const f16 mask = valid ? (f16)0.f : (f16)(-__builtin_inff());
          *reinterpret_cast<uint4*>(&tile[r * kS + kZ + 8]) =
              make_uint4(__builtin_bit_cast(uint32_t, f16x2{(f16)0.f, mask}),
                         __builtin_bit_cast(uint32_t, f16x2{(f16)1.f, (f16)0.f}), 0, 0);
        }
        return;
      }
      // content codes (this thread's share): consecutive lanes write consecutive 16-byte (C4) or
      // 32-byte (C2) runs
      unpack_content<BITS_C, 0, GE::CQ>(tile, ft, R.c);
      // RoPE-key codes: dword ft holds channels 8 (ft % 8) .. +7 of token ft / 8
      *reinterpret_cast<uint4*>(&tile[(ft >> 3) * kS + kDc + 8 * (ft & 7)]) = unpack4(R.r);
      // metadata (s | z << 16) of token r = ft % 32: group ft / 32, and group 8 for threads < 32
      const int r = ft & 31;
      const int tok = (page0 + (t >> 1)) * kPageTokens + (t & 1) * kT + r;
      const bool valid = tok >= p_lo && tok < p_hi;
      {
        const int g = ft >> 5;
        const float sc = valid ? bf16f(R.m[0] & 0xFFFFu) : 0.f;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(sc >= pv_hi);
        echg = 0;
        if (hit) {  // rare: some scale of the tile reached 2^(pv_e + 6) (or the first nonzero scale)
          float hm = sc;  // maximum over the half wave (the group's 32 tokens)
#pragma unroll
          for (int d = 1; d < 32; d <<= 1) hm = fmaxf(hm, __shfl_xor(hm, d, 64));
          if (hm >= pv_hi) {  // (a normal number: pv_hi >= 2^-126)
            pv_e = min(max(((__float_as_int(hm) >> 23) & 0xFF) - 127 - 5, -100), 120);
            pv_inv = __builtin_ldexpf(1.f, -pv_e);
            pv_hi = __builtin_ldexpf(1.f, pv_e + 6);
          }
          if (r == 0) sm.pve[sl][g] = pv_e;
          echg = 2;
        }
        sm.sq[sl][g][sq_pos(r)] = sc * c_log2;
        sm.svh[sl][g][pv_pos(r)] = (f16)(sc * pv_inv);
        tile[r * kS + kZ + g] = (f16)(valid ? bf16f(R.m[0] >> 16) : 0.f);
      }
      if (ft < kT) {
        const float sc = valid ? bf16f(R.m[1] & 0xFFFFu) : 0.f;
        sm.sq[sl][8][sq_pos(r)] = sc * c_log2;
        const f16 z8 = (f16)(valid ? bf16f(R.m[1] >> 16) : 0.f);
        const f16 mask = valid ? (f16)0.f : (f16)(-__builtin_inff());  // score mask, column kZ + 9
        // column kZ + 10 holds 1: the PV waves' zero-term MFMA sums each head's probabilities there
        *reinterpret_cast<uint4*>(&tile[r * kS + kZ + 8]) =
            make_uint4(__builtin_bit_cast(uint32_t, f16x2{z8, mask}),
                       __builtin_bit_cast(uint32_t, f16x2{(f16)1.f, (f16)0.f}), 0, 0);
      }
    };

    // queries: A operand of QK 16x16x32 (lane: head head0 + 16w + L16, positions 32 ks + 8 G + j)
    f16x8 qreg[18];
    f16x8 qz;
    auto load_queries = [&]() {
      float qs[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) qs[g] = 0.f;
      const uint16_t* qh = p.q + ((int64_t)b * p.heads + head0 + 16 * w + L16) * kD;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qh + 32 * ks + 8 * G);
        const uint4 hv = ks < 16 ? bf16_chunk_to_f16<BITS_C>(raw) : bf16_chunk_to_f16<4>(raw);
        qreg[ks] = __builtin_bit_cast(f16x8, hv);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += (float)qreg[ks][j];
        qs[ks < 16 ? ks / 2 : 8] += sum;
      }
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        qs[g] += __shfl_xor(qs[g], 16, 64);
        qs[g] += __shfl_xor(qs[g], 32, 64);
        qs[g] *= c_log2;
      }
      // zero-term step, k = 8 G + j: G0 hi(qsum_j), G2 lo(qsum_j) against z_j; G1 / G3 hi / lo of
      // qsum_8 in slot j = 0 against z_8, and 1 in slot j = 1 against the token's score mask (0, or
      // -inf for a token outside the item: twice -inf is -inf); the other slots meet zero columns.
      // (Lane groups 0 and 1 share LDS read passes: reading different column blocks keeps them on
      // distinct banks.)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (G & 1) == 0 ? qs[j] : (j == 0 ? qs[8] : 0.f);
        const f16 hi = (f16)x;
        const f16 lo = (f16)(x - (float)hi);
        qz[j] = (G & 1) && j == 1 ? (f16)1.f : (G >> 1) ? lo : hi;
      }
    };
    float m_run[4];  // heads .. + 4G + i (the lane's D rows)
    float m_thr[4], m_sub[4];   // m_run + kRescale, and m_run as subtracted from scores (0 while -inf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_thr[i] = -__builtin_inff();
      m_sub[i] = 0.f;
      m_run[i] = -__builtin_inff();
    }
    // QK and softmax of tile k; probabilities to probT[k % 2]
    auto qk_step = [&](int k) {
      if (k >= n_tiles) return;
      const int sl = k % kSlots, pb = k & 1;
      const lds_ptr<f16> tb = lds_opaque(&sm.tile[sl][0]);
      // lane (token L16 of each 16-token block, heads .. + 4G + i)
      f32x4 S[2];
      {
        const lds_ptr<float> sqp = lds_opaque(&sm.sq[sl][0][0]) + 2 * L16;
        const lds_ptr<f16> k0 = tb + L16 * kS + 8 * G;
        const lds_ptr<f16> k1 = k0 + 16 * kS;
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        // software pipeline: the tile operands and scales of group g + kAhead are requested
        // before group g multiplies (the scheduling fences keep the requests in place)
        constexpr int kAhead = 3;
        f16x8 kf[kAhead][4];
        f32x2 scf[kAhead];
        // groups in the order 8 (RoPE key), 0, 1, .., 7: the RoPE-key product is requested and
        // issued first
        auto grp = [](int i) { return i == 0 ? kGroups - 1 : i - 1; };
        auto request = [&](int i) {
          const int g = grp(i);
          kf[i % kAhead][0] = lds_load<f16x8>(k0 + 64 * g);
          kf[i % kAhead][1] = lds_load<f16x8>(k1 + 64 * g);
          kf[i % kAhead][2] = lds_load<f16x8>(k0 + 64 * g + 32);
          kf[i % kAhead][3] = lds_load<f16x8>(k1 + 64 * g + 32);
          scf[i % kAhead] = lds_load<f32x2>(sqp + g * kT);
        };
#pragma unroll
        for (int i = 0; i < kAhead; ++i) request(i);
#pragma unroll
        for (int i = 0; i < kGroups; ++i) {
          const int g = grp(i), r = i % kAhead;
          const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
          f32x4 c0 = mfma16(qreg[2 * g], kf[r][0], z4);
          f32x4 c1 = mfma16(qreg[2 * g], kf[r][1], z4);
          c0 = mfma16(qreg[2 * g + 1], kf[r][2], c0);
          c1 = mfma16(qreg[2 * g + 1], kf[r][3], c1);
          const f32x2 sc = scf[r];
          __builtin_amdgcn_sched_barrier(0);
          if (i + kAhead < kGroups) request(i + kAhead);
          __builtin_amdgcn_sched_barrier(0);
          s[0] += sc[0] * c0;
          s[1] += sc[1] * c1;
        }
        // zero terms of all nine groups
        const int zc = kZ + 8 * (G & 1);
        const f16x8 zr0 = lds_load<f16x8>(tb + L16 * kS + zc);
        const f16x8 zr1 = lds_load<f16x8>(tb + (16 + L16) * kS + zc);
        S[0] = mfma16(qz, zr0, s[0]);
        S[1] = mfma16(qz, zr1, s[1]);
      }
      if (!packed && p.q_len > 1) {
        // several query tokens: this wave's query (its 16 heads belong to one) sees the first
        // n_vis tokens; the ones it does not see are all in the recent window (bf16 items)
        const int n_vis = N - (p.q_len - 1 - (head0 + 16 * w) / p.heads_per_query);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int j = jb + k * kT + 16 * blk + L16;
          const int tok = j < ns ? j : rstart + (j - ns);
          if (tok >= n_vis) S[blk] = f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
        }
      }
      // online softmax; a head's running max is refreshed only when one of its scores
      // exceeds it by more than kRescale
      bool need = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) need |= (S[0][i] > m_thr[i]) | (S[1][i] > m_thr[i]);
      const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
      float alpha[4] = {1.f, 1.f, 1.f, 1.f};
      if (any) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float mx = row16_max(fmaxf(S[0][i], S[1][i]));
          const float m_new = fmaxf(m_run[i], mx);
          alpha[i] = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
          m_run[i] = m_new;
          m_thr[i] = m_new + kRescale;
          m_sub[i] = m_new == -__builtin_inff() ? 0.f : m_new;
        }
      }
      f16x4 pz[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(S[0][i] - m_sub[i]);
        const float e1 = __builtin_amdgcn_exp2f(S[1][i] - m_sub[i]);
        pz[0][i] = (f16)e0;
        pz[1][i] = (f16)e1;
      }
      const int hc = 16 * w + 4 * G;  // first head column of the lane's rows
      *reinterpret_cast<f16x4*>(&sm.probT[pb][p_row(L16)][hc]) = pz[0];
      *reinterpret_cast<f16x4*>(&sm.probT[pb][p_row(16 + L16)][hc]) = pz[1];
      if (L16 == 0) *reinterpret_cast<f32x4*>(&sm.alpha[pb][hc]) = f32x4{alpha[0], alpha[1], alpha[2], alpha[3]};
      if (lane == 0) sm.resc[pb][w] = (any ? 1 : 0) | echg;  // echg: set by the fill of tile k
    };

    if (packed) {
      // tile t lives in R(t % 3); step k requests tile k + 3 into the registers tile k held, scores
      // tile k and unpacks tile k + 1 (the waits for its loads, two batches deep, come from the compiler)
      TileRegs<BITS_C> R0, R1, R2;
      auto step = [&](int k, TileRegs<BITS_C>& next, const TileRegs<BITS_C>& cur) {
        load(k + 3, next);
        qk_step(k);
        if (k + 1 < n_tiles) fill(k + 1, cur);
        __syncthreads();
      };
      load(0, R0);
      load(1, R1);
      load(2, R2);
      load_queries();
      fill(0, R0);
      __syncthreads();  // first tile unpacked
      for (int k = 0; k < n_steps; k += 3) {
        step(k, R0, R1);
        step(k + 1, R1, R2);
        step(k + 2, R2, R0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no loads left in flight at exit
      if (bad_pages && lane == 0) atomicAdd(p.plan_hdr + kHdrBadPages, bad_pages);
    } else {
      const TileRegs<BITS_C> none{};
      BfRegs X;
      load_queries();
      if (n_tiles > 0) {
        bf_load(0, X, std::integral_constant<int, kBfQK>{});
        bf_store(0, X, std::integral_constant<int, kBfQK>{});
        fill(0, none);
      }
      __syncthreads();  // first tile converted
      for (int k = 0; k < n_steps; ++k) {
        const bool next = k + 1 < n_tiles;
        if (next) bf_load(k + 1, X, std::integral_constant<int, kBfQK>{});
        qk_step(k);
        if (next) {
          bf_store(k + 1, X, std::integral_constant<int, kBfQK>{});
          fill(k + 1, none);
        }
        __syncthreads();
      }
    }
    // running max of the heads of this wave (their sums come from the PV waves)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (L16 == 0) {
        const int hh = 16 * w + 4 * G + i;
        if (direct) x_ml[2 * hh] = m_run[i];
        else p.ws_ml[2 * (row0 + hh)] = m_run[i];
      }
    }
    if (direct) {
      if (tid == 0) atomicAdd(p.plan_hdr + kHdrDirect, 1);
      __syncthreads();  // (the PV waves' matching barrier is in their epilogue)
    }
  } else {
    // ============ PV waves: content groups 2v, 2v + 1 for all 64 heads ============
    const int v = w - 4;
    // rows z index 4G + i, column head 16v + L16: sum_t p z_i for i < 8; row 10 (G = 2, register 2)
    // meets the ones column: the head's sum of probabilities
    f32x4 oz = {0.f, 0.f, 0.f, 0.f};
    f32x16 O[2][4];                    // [head block][channel block]
    int cur_e[2] = {0, 0};             // O[.][2 gi + c] holds sum_t code * p * s * 2^-cur_e[gi]
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) O[hb][cb] = f32x16{};
    // accumulate tile k - 1 (ring slot (k - 1) % 3, probabilities of step k - 1)
    auto pv_step = [&](int k) {
      if (k >= 1 && k <= n_tiles) {
        const int sl = (k - 1) % kSlots, pb = (k - 1) & 1;
        const lds_ptr<f16> tb = lds_opaque(&sm.tile[sl][0]);
        const lds_ptr<int> rf = lds_opaque(&sm.resc[pb][0]);
        const lds_ptr<f16> ptb = lds_opaque(&sm.probT[pb][0][0]);
        // request every operand of the step before multiplying (the fence keeps them together)
        // zero-term sums for heads 16v + L16 (A: z rows from the zero-term columns, k: tokens
        // zt0 | zt1; B: the same tokens' probabilities)
        const int zt0 = pv_token((G >> 1) + 4 * (G & 1), L16 >> 2), zt1 = pv_token((G >> 1) + 2 + 4 * (G & 1), L16 >> 2);
        const lds_ptr<f16> za = tb + kZ + 4 * (L16 & 3), pa = ptb + 16 * v + 4 * (L16 & 3);
        const f16x8 zA = cat(lds_tr4(za + zt0 * kS), lds_tr4(za + zt1 * kS));
        const f16x8 zP = cat(lds_tr4(pa + p_row(zt0) * kPT), lds_tr4(pa + p_row(zt1) * kPT));
        const lds_ptr<f16> svw = lds_opaque(&sm.svh[sl][2 * v][0]);
        f16x8 A[2][4], P[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // k slots of this half: the tokens of sets ks + 4 half, then ks + 2 + 4 half
          const int t0 = pv_token(ks + 4 * half, (lane & 15) >> 2), t1 = pv_token(ks + 2 + 4 * half, (lane & 15) >> 2);
          const int csel = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          const lds_ptr<f16> va = tb + 128 * v + csel, pbp = ptb + csel;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) A[ks][cb] = cat(lds_tr4(va + t0 * kS + 32 * cb), lds_tr4(va + t1 * kS + 32 * cb));
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) P[ks][hb] = cat(lds_tr4(pbp + p_row(t0) * kPT + 32 * hb), lds_tr4(pbp + p_row(t1) * kPT + 32 * hb));
        }
        // the refresh flags are read with the operands, so one wait covers both
        if (rf[0] | rf[1] | rf[2] | rf[3]) {
          float ef[2] = {1.f, 1.f};
          if (rf[v] & 2) {  // this wave's groups 2v, 2v + 1 changed their PV scale exponent
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
              const int ne = sm.pve[sl][2 * v + gi];
              ef[gi] = __builtin_ldexpf(1.f, cur_e[gi] - ne);
              cur_e[gi] = ne;
            }
          }
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const float a = sm.alpha[pb][32 * hb + l32];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) O[hb][cb] *= a * ef[cb >> 1];
          }
          oz *= sm.alpha[pb][16 * v + L16];
        }
        __builtin_amdgcn_sched_barrier(0);
        oz = mfma16(zA, zP, oz);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const f16x8 sv = lds_load<f16x8>(svw + gi * kT + 16 * ks + 8 * half);
            const f16x8 b0 = P[ks][0] * sv, b1 = P[ks][1] * sv;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const int cb = 2 * gi + c;
              O[0][cb] = mfma32(A[ks][cb], b0, O[0][cb]);
              O[1][cb] = mfma32(A[ks][cb], b1, O[1][cb]);
            }
          }
      }
    };

    if (packed) {
      // the PV threads load and unpack the content dwords the QK threads leave (same three-tile
      // register ring: step k requests tile k + 3, unpacks tile k + 1, accumulates tile k - 1)
      const int pt = tid - 256;
      cint* bt = (cint*)(uintptr_t)(p.block_table + (int64_t)slot * p.max_pages);
      auto pload = [&](int t, PVRegs<BITS_C>& R) {
        t = min(t, n_tiles - 1);
        int uncounted = 0;  // (the QK waves count the same reads)
        const uint8_t* base = p.pages + page_of(p, bt, page0 + (t >> 1), &uncounted) * (int64_t)GE::PB;
        const uint32_t* srcC = reinterpret_cast<const uint32_t*>(base + (t & 1) * kT * GE::CB);
#pragma unroll
        for (int i = 0; i < GE::CPT - GE::CQ; ++i) R.c[i] = srcC[pt + 256 * (GE::CQ + i)];
      };
      auto pfill = [&](int t, const PVRegs<BITS_C>& R) {
        unpack_content<BITS_C, GE::CQ, GE::CPT - GE::CQ>(&sm.tile[t % kSlots][0], pt, R.c);
      };
      auto step = [&](int k, PVRegs<BITS_C>& next, const PVRegs<BITS_C>& cur) {
        pload(k + 3, next);
        // the unpack first: its VALU work meets the QK waves' MFMAs at the start of the step, and
        // the PV MFMAs meet the QK waves' softmax and unpack at its end
        if (k + 1 < n_tiles) pfill(k + 1, cur);
        pv_step(k);
        __syncthreads();
      };
      PVRegs<BITS_C> R0, R1, R2;
      pload(0, R0);
      pload(1, R1);
      pload(2, R2);
      pfill(0, R0);
      __syncthreads();  // first tile unpacked
      for (int k = 0; k < n_steps; k += 3) {
        step(k, R0, R1);
        step(k + 1, R1, R2);
        step(k + 2, R2, R0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no loads left in flight at exit
    } else {
      BfRegs X;
      if (n_tiles > 0) {
        bf_load(0, X, std::integral_constant<int, kBfPV>{});
        bf_store(0, X, std::integral_constant<int, kBfPV>{});
      }
      __syncthreads();  // first tile converted
      for (int k = 0; k < n_steps; ++k) {
        const bool next = k + 1 < n_tiles;
        if (next) bf_load(k + 1, X, std::integral_constant<int, kBfPV>{});
        pv_step(k);
        if (next) bf_store(k + 1, X, std::integral_constant<int, kBfPV>{});
        __syncthreads();
      }
    }
    if (direct) {
      if (G < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x_z[(16 * v + L16) * 8 + 4 * G + i] = oz[i];
      }
      if (G == 2) x_ml[2 * (16 * v + L16) + 1] = oz[2];
      __syncthreads();  // every head's max, sum and zero-term sums are in place
      if (G == 2 && p.lse) {
        const float mh = x_ml[2 * (16 * v + L16)];
        p.lse[orow0 + 16 * v + L16] =
            mh == -__builtin_inff() ? -__builtin_inff() : (mh + __log2f(oz[2])) * 0.69314718055994531f;
      }
    } else if (G == 2) {
      p.ws_ml[2 * (row0 + 16 * v + L16) + 1] = oz[2];
    }
    // unnormalised partial output and zero-term sums (direct: the final bf16 outputs of the head
    // rows, (sum + zero term of the group) / sum of probabilities).  Registers 4a .. 4a + 3 of lanes l and l ^ 32
    // hold the 8 channels 8 (16 v + 4 cb + a) + 0..7 between them, in the unpacking order; each
    // lane takes two values from the other, so that the lower half holds channels 0..3 and the
    // upper half channels 4..7, written as one 16-byte store.
    const bool odd = half;
    const float e2[2] = {__builtin_ldexpf(1.f, cur_e[0]), __builtin_ldexpf(1.f, cur_e[1])};  // undo 2^-E_g
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hh = 32 * hb + l32;
      float* dh = p.ws_o + (row0 + hh) * kDc;
      uint16_t* oh = p.out + (orow0 + hh) * kDc;
      float inv = 0.f, zg[2] = {0.f, 0.f};  // (direct) 1 / sum, zero terms of groups 2v, 2v + 1
      if (direct) {
        inv = x_ml[2 * hh] == -__builtin_inff() ? 0.f : 1.f / x_ml[2 * hh + 1];
        zg[0] = x_z[hh * 8 + 2 * v];
        zg[1] = x_z[hh * 8 + 2 * v + 1];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 x = f32x4{O[hb][cb][4 * a], O[hb][cb][4 * a + 1], O[hb][cb][4 * a + 2], O[hb][cb][4 * a + 3]} *
                          e2[cb >> 1];
          f32x4 r;
          if (BITS_C == 4) {  // lower lane: channels 0 2 4 6, upper lane: 1 3 5 7
            const float rx = __shfl_xor(odd ? x[0] : x[2], 32, 64);
            const float ry = __shfl_xor(odd ? x[1] : x[3], 32, 64);
            r = odd ? f32x4{rx, x[2], ry, x[3]} : f32x4{x[0], rx, x[1], ry};
          } else {            // lower lane: channels 0 4 1 5, upper lane: 2 6 3 7
            const float rx = __shfl_xor(odd ? x[0] : x[1], 32, 64);
            const float ry = __shfl_xor(odd ? x[2] : x[3], 32, 64);
            r = odd ? f32x4{rx, ry, x[1], x[3]} : f32x4{x[0], x[2], rx, ry};
          }
          const int c0 = 8 * (16 * v + 4 * cb + a) + 4 * half;  // channels c0 .. c0 + 3, group 2v + cb / 2
          if (direct) store_bf16x4(oh + c0, (r + zg[cb >> 1]) * inv);
          else *reinterpret_cast<f32x4*>(dh + c0) = r;
        }
    }
    if (G < 2 && !direct) {
      const int64_t hrow = row0 + 16 * v + L16;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.ws_z[hrow * 8 + 4 * G + i] = oz[i];
    }
  }
}

template <int BITS_C>
hipError_t prepare64() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(decode64_kernel<BITS_C>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem64<BITS_C>));
}

template <int BITS_C>
hipError_t launch64(const DecodeParams& p, hipStream_t stream) {
  const int64_t blocks = ((int64_t)p.max_items + 7) / 8 * 8 * p.head_groups;
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(decode64_kernel<BITS_C>), dim3((unsigned)blocks),
                         dim3(kThreads), args, sizeof(Smem64<BITS_C>), stream);
}

}  // namespace

hipError_t prepare_decode64(const DecodeParams&, int bits_c) {
  if (bits_c == 4) return prepare64<4>();
  if (bits_c == 2) return prepare64<2>();
  return hipErrorInvalidValue;
}

hipError_t launch_decode64(const DecodeParams& p, int bits_c, hipStream_t stream) {
  if (bits_c == 4) return launch64<4>(p, stream);
  if (bits_c == 2) return launch64<2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
