// Split-KV low-bit MLA decode for groups of 16 query heads on gfx950 (CDNA4).
//
// Same computation as decode64.hip (QuantMLA pages: ai.info summary, "Key
// Contributions", item 4; onedev.kr review, "How it is used"): one global
// softmax over all valid tokens, sink / recent tokens from bf16, all others
// from their packed copies, output aggregated over the content latent.
//
// With 16 heads per latent the decode is HBM-bound: every packed code feeds a
// single 16-head MFMA block.  One workgroup of 8 waves (two per SIMD) per
// (sequence, split, 16-head group), working as four independent pairs.  Pair r
// (waves r and r + 4) owns rows 16r..16r+15 of every page of the split; the
// pair's two waves split the work by role and run concurrently, so one wave's
// stalls are covered by other waves' work:
//  - the QK wave loads, for each 16-token block of the pair, its lanes' packed
//    words straight from HBM into registers three blocks ahead (the K-step
//    words of the lane's token row for every group, and the token's nine
//    metadata words).  QK: MFMA 16x16x32 f16, queries as the A operand, the
//    exact codes of the block as the B operand (nibbles / crumbs become fp8
//    bytes whose e4m3 value is code * 2^-9, converted with a 2^9 scale); each
//    lane owns one token, so a group's fp32 scale is one scalar; the zero
//    terms of all nine groups go through one more MFMA.  Online softmax in the
//    log2 domain with a lazily refreshed running max.  The unpacked content
//    codes, zeros, PV scales and fp16 probabilities of block t go to the pair's
//    tile buffer t % 2;
//  - the PV wave takes the block's operands from that buffer (transposed
//    reads, ds_read_b64_tr_b16) into registers, releases it, and accumulates
//    MFMA 16x16x16 f16 of the codes against p * s_g, plus sum_t p_t z_g,t.
// The two waves hand blocks over through LDS sequence flags: the QK wave
// publishes block t once its buffer is written, and writes block t only after
// the PV wave has released block t - 2 (two buffers), so it runs up to a block
// ahead.  Every wait is bounded, so a broken handshake gives wrong values,
// never a hang; a wait that gives up is counted in the workspace header.  The four pairs' partials are merged through LDS at the end;
// the split's partial stays unnormalised with its running max and sum for the
// combine.
#include <algorithm>
#include <cstddef>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

constexpr int kPairs = 4;             // QK waves 0..3, PV waves 4..7 (pair r: waves r and r + 4)
constexpr int kThreads = 128 * kPairs;
constexpr int kB = 16;                // tokens per block (one pair's rows of a page)
constexpr int kAhead = 3;             // blocks a QK wave holds in registers (block t and two more in flight)
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
  int resc;           // bit 0: apply alpha before this block; bit 1: the PV scale exponent changed
  int pv_exp;         // E: the block's PV scales are fp16(s * 2^-E) (valid when bit 1 of resc is set)
  int pad[2];
};
union __align__(16) Tiles16 {
  PairTiles pt[kPairs][2];
  struct {                   // merge of the pairs' partials at the end (two pairs at a time)
    float o[2][16][kDc];
    float m[kPairs][16], l[kPairs][16];
    float z[kPairs][16][8];
  } mg;
};

__device__ __forceinline__ f32x4 mfma32k(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 4, 64));
  return fmaxf(v, __shfl_xor(v, 8, 64));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  return v + __shfl_xor(v, 8, 64);
}

// Handshake flags live in an LDS object of their own, read and written as volatile words.
typedef __attribute__((address_space(3))) volatile int lds_vint;
// Returns 1 when the wait gave up after `spin` polls (counted into the workspace header).
__device__ __forceinline__ int wait_at_least(lds_vint* flag, int target, int spin) {
  for (int i = 0; i < spin; ++i) {
    if (__builtin_amdgcn_readfirstlane(*flag) >= target) return 0;
    __builtin_amdgcn_s_sleep(1);
  }
  return 1;
}
// publish a flag value once this wave's earlier LDS writes have completed
__device__ __forceinline__ void signal(lds_vint* flag, int value, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) *flag = value;
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
  constexpr int oR = (int)offsetof(PairTiles, resc), oE = (int)offsetof(PairTiles, pv_exp);
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
  const int o_pe = pb0 + oE;
  __syncthreads();  // flags initialised

  auto& mg = s_tiles.mg;
  const int spin = p.spin_limit;
  int give_ups = 0, bad_pages = 0;  // (uniform across the wave)
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
    // PV scale normaliser of a packed item: its PV scales go to the tile as fp16(s * 2^-pv_e), with
    // pv_e raised (never lowered) so that the largest scale seen so far sits in [2^5, 2^6); with
    // probabilities <= 2^8 (lazy max refresh) every product p * s * 2^-pv_e stays below 2^14.
    int pv_e = 0, ebit = 0;                 // ebit: 2 when the current block raised pv_e
    float pv_inv = 1.f, pv_hi = 0x1p-126f;  // 2^-pv_e; raise when a scale reaches pv_hi = 2^(pv_e + 6)
    // smax: the larger of the two PV scales this lane writes (groups 2G, 2G + 1 of token L16), so
    // the maximum over the wave is the block's largest scale
    auto pv_scale_check = [&](float smax) {
      ebit = 0;
      if (__builtin_amdgcn_ballot_w64(smax >= pv_hi) == 0) return;
      float m = smax;  // (some lane holds a scale >= pv_hi >= 2^-126: the maximum is a normal number)
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      const int bits = __builtin_amdgcn_readfirstlane(__float_as_int(m));
      pv_e = min(max(((bits >> 23) & 0xFF) - 127 - 5, -100), 120);
      pv_inv = __builtin_ldexpf(1.f, -pv_e);
      pv_hi = __builtin_ldexpf(1.f, pv_e + 6);
      ebit = 2;
    };
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
    auto publish = [&](f32x4 S, int t, int rbits, int so) {
      f16x4 pz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mu = m_run[i] == -__builtin_inff() ? 0.f : m_run[i];
        const float e = __builtin_amdgcn_exp2f(S[i] - mu);
        l_part[i] += e;
        pz[i] = (f16)e;
      }
      *reinterpret_cast<lds_ptr<f16x4>>(tb + (o_pwr + so)) = pz;
      if (lane == 0) {
        *reinterpret_cast<lds_ptr<int>>(tb + (o_rs + so)) = rbits;
        if (rbits & 2) *reinterpret_cast<lds_ptr<int>>(tb + (o_pe + so)) = pv_e;
      }
      signal(fl + 0, t, lane);
    };
    // the QK of one block from K-step words kw(g) (C4 / RoPE: two dwords, C2: one), its scales and
    // zeros in mw (bf16 s | z << 16, 0 for masked tokens); writes the V, Z and SV tiles, returns S
    // (rows heads 4G + i, column token L16)
    auto block_qk = [&](auto&& kw, auto&& kf16, const uint32_t* mw, bool valid, bool codes, int so) -> f32x4 {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kGroups; ++i) {  // groups 8 (RoPE key), 0, 1, .., 7: the RoPE-key product first
        const int g = i == 0 ? kGroups - 1 : i - 1;
        f16x8 k0, k1;
        if (codes) {
          const u32x2 v = kw(g);
          if (g == 8 || BITS_C == 4) {
            k0 = __builtin_bit_cast(f16x8, unpack4(v.x));
            k1 = __builtin_bit_cast(f16x8, unpack4(v.y));
          } else {
            uint4 x0, x1;
            unpack2(v.x, x0, x1);
            k0 = __builtin_bit_cast(f16x8, x0);
            k1 = __builtin_bit_cast(f16x8, x1);
          }
        } else {
          k0 = kf16(g, 0);
          k1 = kf16(g, 1);
        }
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
        if (codes) pv_scale_check(fmaxf(s0, s1));  // (bf16 items keep pv_inv = 1)
        *reinterpret_cast<lds_ptr<f16>>(tb + (o_svw + so + 64 * G)) = (f16)(s0 * pv_inv);
        *reinterpret_cast<lds_ptr<f16>>(tb + (o_svw + so + 64 * G + 32)) = (f16)(s1 * pv_inv);
        if (G == 0) {
          *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_zwr + so)) = zlo;
          *reinterpret_cast<lds_ptr<f16>>(tb + (o_zwr + so + 16)) = z8;
        }
      }
      return mfma32k(qz, zf, s * c_log2) + (valid ? 0.f : -__builtin_inff());
    };

    if (packed) {
      // page ids through the constant address space: uniform index, so scalar loads
      typedef __attribute__((address_space(4))) const int32_t cint;
      cint* bt = (cint*)(uintptr_t)(p.block_table + (int64_t)slot * p.max_pages + page0);
      // The packed bytes of one block this lane needs, straight from HBM into registers: its token
      // row's K-step words of every group (C4 / RoPE: two dwords, C2: one) and the token's nine
      // metadata words.  Every call issues the same loads (block index clamped), so the
      // compiler's count of loads in flight stays exact.
      struct BlockRegs {
        u32x2 kv[kGroups];
        uint32_t mw[kGroups];
      };
      auto load = [&](int t, BlockRegs& R) {
        int pg = bt[min(t, last)];
        if (pg < 0 || pg >= p.num_pages) {  // contract violation: wrong values, no fault; counted
          pg = 0;
          ++bad_pages;
        }
        const uint8_t* base = p.pages + (int64_t)pg * GE::PB;
        const uint8_t* crow = base + row * GE::CB + (BITS_C == 4 ? 8 : 4) * G;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          if (BITS_C == 4) R.kv[g] = *reinterpret_cast<const u32x2*>(crow + 32 * g);
          else R.kv[g] = u32x2{*reinterpret_cast<const uint32_t*>(crow + 16 * g), 0u};
        }
        R.kv[8] = *reinterpret_cast<const u32x2*>(base + GE::ROPE0 + row * (kDr / 2) + 8 * G);
        const uint32_t* mrow = reinterpret_cast<const uint32_t*>(base + GE::META0 + row * 4 * kGroups);
#pragma unroll
        for (int g = 0; g < kGroups; ++g) R.mw[g] = mrow[g];
      };
      auto step = [&](int t, BlockRegs& R) {
        if (t <= last) {
          const int tok = (page0 + t) * kPageTokens + row;
          const bool valid = tok >= p_lo && tok < p_hi;
          uint32_t mw[kGroups];
#pragma unroll
          for (int g = 0; g < kGroups; ++g) mw[g] = valid ? R.mw[g] : 0u;
          auto kw = [&](int g) -> u32x2 { return R.kv[g]; };
          auto none = [&](int, int) { return f16x8{}; };
          const int so = (t & 1) * kPT;
          give_ups += wait_at_least(fl + 1, t - 2, spin);  // the PV wave has read buffer t % 2 (block t - 2)
          const f32x4 S = block_qk(kw, none, mw, valid, true, so);
          const bool resc = needs_refresh(S);
          if (resc) refresh(S, so);
          publish(S, t, (resc ? 1 : 0) | ebit, so);
        }
        load(t + kAhead, R);  // the registers of block t now take block t + 3
      };
      BlockRegs R0, R1, R2;
      load(0, R0);
      load(1, R1);
      load(2, R2);
      load_queries();
      for (int t = 0; t <= last; t += 3) {
        step(t, R0);
        step(t + 1, R1);
        step(t + 2, R2);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no loads left in flight at exit
    } else {
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
        auto none = [&](int) { return u32x2{0u, 0u}; };
        const int so = (t & 1) * kPT;
        give_ups += wait_at_least(fl + 1, t - 2, spin);  // buffer t % 2 is free
        const f32x4 S = block_qk(none, kf16, mw, valid, false, so);
        const bool resc = needs_refresh(S);
        if (resc) refresh(S, so);
        publish(S, t, resc ? 1 : 0, so);
      }
    }
    if (lane == 0 && give_ups) atomicAdd(p.plan_hdr + kHdrGiveUps, give_ups);
    if (lane == 0 && bad_pages) atomicAdd(p.plan_hdr + kHdrBadPages, bad_pages);
    // ---- merge: this pair's running max and sum
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
  } else {
    // ============================== PV wave of pair pr ==============================
    f32x4 O[32];  // column head L16, rows channel positions 16 cb + 4G + i
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) O[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oz = {0.f, 0.f, 0.f, 0.f};  // rows z index 4G + i
    int cur_e = 0;                     // O holds sum_t code * p * s * 2^-cur_e (packed items)
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
      const int new_e = __builtin_amdgcn_readfirstlane(lds_load<int>(tb + (o_pe + so)));
      const float alpha = lds_load<float>(tb + (o_al + so + 4 * L16));
      signal(fl + 1, t, lane);
      if (resc) {
        const float a = (resc & 1) ? alpha : 1.f;
        float ae = a;
        if (resc & 2) {  // the PV scales now carry 2^-new_e: bring the sums to that scale
          ae = a * __builtin_ldexpf(1.f, cur_e - new_e);
          cur_e = new_e;
        }
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) O[cb] *= ae;
        oz *= a;
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
    // ---- merge the four pairs' partials (per head: max-shifted sums) and write the split's row
    __syncthreads();  // every wave is done with its tiles; the merge area overlays them
    __syncthreads();  // the QK waves' running maxima and sums are in place
    float M = -__builtin_inff();  // merged max of head L16 (the PV column)
#pragma unroll
    for (int v = 0; v < kPairs; ++v) M = fmaxf(M, mg.m[v][L16]);
    {
      const float mw = mg.m[pr][L16];
      const float f = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      const float fe = f * __builtin_ldexpf(1.f, cur_e);  // undo the PV scale normaliser
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
      const int64_t orow = (int64_t)item * p.heads + head0 + L16;
      float* dst = p.ws_o + orow * kDc;
      // Lanes G and G ^ 1 (lane ^ 16) hold the 8 channels 16 cb + 8 (G >> 1) + 0..7 between them,
      // in the unpacking order; each takes two values from the other so that lane G even holds
      // channels 0..3 and lane G odd channels 4..7, written as one 16-byte store.
      const bool odd = G & 1;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        const f32x4 v = O[cb];
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
        *reinterpret_cast<f32x4*>(dst + 16 * cb + 8 * (G >> 1) + 4 * (G & 1)) = r;
      }
      if (G == 0) {
        float L = 0.f, zs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < kPairs; ++v) {
          const float mv = mg.m[v][L16];
          L += (mv == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mv - M)) * mg.l[v][L16];
#pragma unroll
          for (int g = 0; g < 8; ++g) zs[g] += mg.z[v][L16][g];
        }
        p.ws_ml[2 * orow] = M;
        p.ws_ml[2 * orow + 1] = L;
#pragma unroll
        for (int g = 0; g < 8; ++g) p.ws_z[orow * 8 + g] = zs[g];
      }
    }
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
