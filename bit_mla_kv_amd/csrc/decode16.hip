// Split-KV low-bit MLA decode for groups of 16 query heads on gfx950 (CDNA4).
//
// Same computation as decode64.hip (QuantMLA pages: ai.info summary, "Key
// Contributions", item 4; onedev.kr review, "How it is used"): one global
// softmax over all valid tokens, sink / recent tokens from bf16, all others
// from their packed copies, output aggregated over the content latent.
//
// With 16 heads per latent the decode is HBM-bound: every packed code feeds a
// single 16-head MFMA block, so the waves share nothing while the cache
// streams through.  One workgroup of 4 waves (one per SIMD) per (sequence,
// split, 16-head group); wave w owns rows 16w..16w+15 of every page of the
// split and works through them without workgroup barriers:
//  - the wave's 16-token block of a page (packed codes, RoPE codes, metadata)
//    lands in the wave's own three-zone LDS staging ring straight from HBM
//    (global_load_lds_dwordx4), blocks t+2 and t+3 in flight while t+1 is
//    read.  A token's content row takes one more 16-byte slot than it needs
//    (the loader lanes of that slot are masked off), so the 16 rows start in
//    different banks and a column of them reads conflict-free;
//  - QK: MFMA 16x16x32 f16, queries as the A operand, the exact codes of the
//    block as the B operand, unpacked in registers from the staging ring
//    (nibbles / crumbs become fp8 bytes whose e4m3 value is code * 2^-9,
//    converted with a 2^9 scale; a lane's 8-channel slice of a K step is one
//    packed dword).  Each lane owns one token, so a group's fp32 scale is one
//    scalar applied to the group's own accumulator; the zero terms of all nine
//    groups go through one more MFMA;
//  - online softmax per block, log2 domain, lazily refreshed running max
//    (the refresh is kept out of the block loop);
//  - PV: the unpacked content codes are also written to a per-wave LDS tile
//    and read back transposed (ds_read_b64_tr_b16) as the A operand of MFMA
//    16x16x16 f16 against p * s_g; one more MFMA accumulates sum_t p_t z_g,t.
//  - software pipeline: PV of block t and QK of block t+1 run fused group by
//    group, the V-tile columns of a group read for block t before block t+1
//    overwrites them, so the MFMAs and unpacking of both blocks interleave.
// The four waves' partials are merged through LDS at the end; the split's
// partial stays unnormalised with its running max and sum for the combine.
#include <algorithm>
#include <cstddef>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

constexpr int kW = 4;             // waves per workgroup
constexpr int kThreads = 64 * kW;
constexpr int kB = 16;            // tokens per block (one wave's rows of a page)
constexpr int kZones = 3;         // staging ring depth per wave
constexpr int kSV = 528;          // V tile row stride (halves): conflict-free b128 row writes and transposed reads
constexpr int kPS = 16;           // probability / zero row stride (halves), rows are tokens
constexpr float kRescale = 8.0f;  // lazy max refresh threshold, log2 units

template <int BITS_C>
struct Geo {
  static constexpr int CB = kDc * BITS_C / 8;                              // content bytes per token
  static constexpr int PB = kPageTokens * (CB + kDr / 2 + 4 * kGroups);   // page bytes
  static constexpr int ROPE0 = kPageTokens * CB;
  static constexpr int META0 = kPageTokens * (CB + kDr / 2);
  // One block in a staging zone: content rows, RoPE rows, metadata rows.  A content row of CU
  // 16-byte units sits in RS = CU + 1 slots (the last one left unwritten), so the rows of the 16
  // tokens start in different LDS banks and a column of units is read without bank conflicts.
  static constexpr int CU = CB / 16;
  static constexpr int RS = CU + 1;
  static constexpr int CI = (kB * RS + 63) / 64;  // content staging instructions (64 slots each)
  static constexpr int SC = CI * 1024;
  static constexpr int SR = kB * kDr / 2;
  static constexpr int SM = kB * 4 * kGroups;
  static constexpr int SZ = SC + SR + SM;
  static constexpr int LOADS = CI + 2;  // staging instructions per block and wave (content, RoPE, metadata)
  static_assert(SR <= 1024 && SM <= 1024, "staging split assumes these sizes");
};

// Per-wave tiles.  They live in an LDS object of their own, apart from the staging ring that the
// HBM-to-LDS loads write, so the compiler can tell the two apart and lets the transposed tile
// reads run while staging loads are still in flight.
struct __align__(16) WaveTiles {
  f16 V[kB][kSV];     // exact content codes of the current block [token][channel position]
  f16 P[kB][kPS];     // fp16 probabilities [token][head]
  f16 Z[kB][kPS];     // fp16 zeros [token][z_0..z_7, 0 x 8]
  f16 SV[8][kB];      // fp16 PV group scales [group][token]
};
union __align__(16) Tiles16 {
  WaveTiles wt[kW];
  struct {                   // merge of the waves' partials at the end (two waves at a time)
    float o[2][16][kDc];
    float m[kW][16], l[kW][16];
    float z[kW][16][8];
  } mg;
};
template <typename T>
__device__ __forceinline__ lds_ptr<T> as_lds(T* p) { return (lds_ptr<T>)p; }

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
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

template <int BITS_C>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode16_kernel(DecodeParams p) {
  using GE = Geo<BITS_C>;
  __shared__ __align__(16) uint8_t s_stage[kW][kZones][GE::SZ];  // packed blocks, block t in zone t % 3
  __shared__ Tiles16 s_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4;
  const int L16 = lane & 15;

  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int hg = kx % p.head_groups;
  const int item = xcd + 8 * (kx / p.head_groups);
  if (item >= min(p.plan_hdr[0], p.max_items)) return;
  const int4 itm = reinterpret_cast<const int4*>(p.items)[item];
  const int b = itm.x;
  const bool packed = itm.w == 0;

  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  const int p_lo = p.n_sink, p_hi = N - p.n_recent;
  const int first_page = p_lo / kPageTokens;
  const int n_pp = p_hi > p_lo ? (p_hi - 1) / kPageTokens - first_page + 1 : 0;
  int n_blocks, page0 = 0, ns = 0, nb = 0, rstart = 0;  // n_blocks: this wave's 16-token blocks
  if (!packed) {
    ns = min(p.n_sink, N);
    rstart = max(p.n_sink, N - p.n_recent);
    nb = ns + max(0, N - rstart);
    n_blocks = (nb + kPageTokens - 1) / kPageTokens;  // bf16 tokens in virtual pages of 64
  } else {
    page0 = itm.y;
    n_blocks = min(min(itm.z, first_page + n_pp - page0), p.max_pages - page0);
    if (n_blocks <= 0) return;
  }
  if (packed && p.num_pages <= 0) return;

  const int head0 = hg * 16;
  const float c_log2 = p.scale_log2e;
  const int row = 16 * w + L16;  // the lane's token row within a page

  // ---- queries: A operand (lane: head head0 + L16; K step (g, h): channels 64g + 16G + 8h .. +7)
  f16x8 qreg[18];
  f16x8 qz;
  {
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
  }

  // ---- state: softmax rows (heads 4G + i); PV accumulators (column head L16, rows channels 4G + i of block cb)
  float m_run[4], l_part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -__builtin_inff();
    l_part[i] = 0.f;
  }
  f32x4 O[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) O[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 oz = {0.f, 0.f, 0.f, 0.f};

  const lds_ptr<f16> vt = as_lds(&s_tiles.wt[w].V[0][0]);
  const lds_ptr<f16> pt = as_lds(&s_tiles.wt[w].P[0][0]);
  const lds_ptr<f16> zt = as_lds(&s_tiles.wt[w].Z[0][0]);
  const lds_ptr<f16> st = as_lds(&s_tiles.wt[w].SV[0][0]);

  // QK of one block: kv(g, h) gives the exact codes (or fp16 values) of K step (g, h) for the lane's
  // token; the content slices also go to the V tile.  Returns S (rows heads 4G + i, column token L16).
  auto block_qk = [&](auto&& kv, const float* s_qk, const float* s_pv, const float* z, float bias) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const f16x8 k0 = kv(g, 0), k1 = kv(g, 1);
      f32x4 c = mfma32k(qreg[2 * g], k0, f32x4{0.f, 0.f, 0.f, 0.f});
      c = mfma32k(qreg[2 * g + 1], k1, c);
      s += s_qk[g] * c;
      if (g < 8) {
        const lds_ptr<f16> dst = vt + L16 * kSV + 64 * g + 16 * G;
        *reinterpret_cast<lds_ptr<f16x8>>(dst) = k0;
        *reinterpret_cast<lds_ptr<f16x8>>(dst + 8) = k1;
      }
      __builtin_amdgcn_sched_barrier(0);  // one group's operands live at a time
    }
    f16x8 zf;
#pragma unroll
    for (int j = 0; j < 8; ++j) zf[j] = (f16)(G < 2 ? z[j] : (j == 0 ? z[8] : 0.f));
    s = mfma32k(qz, zf, s) + bias;
    if (G == 0) {
      f16x8 z8;
#pragma unroll
      for (int j = 0; j < 8; ++j) z8[j] = (f16)z[j];
      *reinterpret_cast<lds_ptr<f16x8>>(zt + L16 * kPS) = z8;
      *reinterpret_cast<lds_ptr<f16x8>>(zt + L16 * kPS + 8) = f16x8{};
#pragma unroll
      for (int g = 0; g < 8; ++g) st[g * kB + L16] = (f16)s_pv[g];
    }
    return s;
  };

  // softmax of one block, probabilities to LDS, then PV over its 16 tokens
  // does some head's score exceed its running max by more than kRescale (wave-uniform)?
  auto needs_refresh = [&](f32x4 S) {
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) need |= S[i] > m_run[i] + kRescale;
    return __builtin_amdgcn_ballot_w64(need) != 0;
  };
  // refresh the running maxima and rescale the accumulators (rare; kept out of the block loop so
  // the accumulators stay in their registers there)
  auto refresh = [&](f32x4 S) {
    {
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m_new = fmaxf(m_run[i], row16_max(S[i]));
        alpha[i] = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
        m_run[i] = m_new;
        l_part[i] *= alpha[i];
      }
      // the PV accumulators hold head L16 in their column; head 4G' + i lives in rows of lanes G'
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha[i], 16 * (L16 >> 2), 64);
      const int sel = L16 & 3;
      const float a = sel == 0 ? a4[0] : sel == 1 ? a4[1] : sel == 2 ? a4[2] : a4[3];
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) O[cb] *= a;
      oz *= a;
    }
  };
  // softmax of one block with the current running maxima, probabilities to LDS, PV over its 16 tokens
  auto softmax_pv = [&](f32x4 S) {
    f16x4 pz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mu = m_run[i] == -__builtin_inff() ? 0.f : m_run[i];
      const float e = __builtin_amdgcn_exp2f(S[i] - mu);
      l_part[i] += e;
      pz[i] = (f16)e;
    }
    *reinterpret_cast<lds_ptr<f16x4>>(pt + L16 * kPS + 4 * G) = pz;
    lds_fence();
    // k = tokens 4G + j: transposed reads of [token][.] rows 4G .. 4G + 3
    const int rsel = 4 * G + (L16 >> 2), csel = 4 * (L16 & 3);
    const f16x4 pb = lds_tr4(pt + rsel * kPS + csel);        // B: head L16
    oz = mfma16k(lds_tr4(zt + rsel * kPS + csel), pb, oz);  // A: z index L16
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const f16x4 bop = pb * lds_load<f16x4>(st + g * kB + 4 * G);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cb = 4 * g + c;  // channel positions 16 cb .. +15
        O[cb] = mfma16k(lds_tr4(vt + rsel * kSV + 16 * cb + csel), bop, O[cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_fence();  // the next block's tile writes come after these reads
  };

  if (packed) {
    // page ids through the constant address space: uniform index, so scalar loads the compiler
    // waits for where the id is used (one step after it is requested)
    typedef __attribute__((address_space(4))) const int32_t cint;
    cint* bt = (cint*)(uintptr_t)(p.block_table + (int64_t)slot * p.max_pages + page0);
    const int last = n_blocks - 1;
    auto page_id = [&](int t) -> int {
      const int pg = bt[min(t, last)];
      return (pg < 0 || pg >= p.num_pages) ? 0 : pg;  // contract violation: wrong values, no fault
    };
    // this lane's source offset and slot use for each content staging instruction
    int coff[GE::CI];
    bool cact[GE::CI];
#pragma unroll
    for (int i = 0; i < GE::CI; ++i) {
      const int sl = 64 * i + lane, tt = sl / GE::RS, u = sl % GE::RS;
      cact[i] = tt < kB && u < GE::CU;
      coff[i] = (16 * w + tt) * GE::CB + 16 * u;
    }
    // block t (page page0 + min(t, last)) into zone t % 3; every block issues GE::LOADS instructions
    auto stage = [&](int t, int pg) {
      const uint8_t* base = p.pages + (int64_t)pg * GE::PB;
      const uint8_t* srcR = base + GE::ROPE0 + 16 * w * (kDr / 2);
      const uint8_t* srcM = base + GE::META0 + 16 * w * 4 * kGroups;
      // The destination goes through an empty asm so that the compiler does not tie these loads
      // to the staging array: its own waits would then hold every read of the array until all
      // staging loads land.  The explicit vmcnt wait before a block is read orders them instead.
      const lds_ptr<uint8_t> zone = lds_opaque(&s_stage[w][t % kZones][0]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of this zone are done
#pragma unroll
      for (int i = 0; i < GE::CI; ++i)
        if (cact[i])
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + coff[i]),
                                           (__attribute__((address_space(3))) void*)(zone + 1024 * i), 16, 0, 0);
      if (lane < GE::SR / 16)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(srcR + 16 * lane),
                                         (__attribute__((address_space(3))) void*)(zone + GE::SC), 16, 0, 0);
      if (lane < GE::SM / 16)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(srcM + 16 * lane),
                                         (__attribute__((address_space(3))) void*)(zone + GE::SC + GE::SR), 16, 0, 0);
    };

    // LDS addressing in the block loop: one base pointer per LDS object plus a byte offset.  The
    // compiler ties an access to its object only through a short chain of address steps, and an
    // access it cannot tie to an object has to wait for every staging load in flight.
    const lds_ptr<uint8_t> sb = (lds_ptr<uint8_t>)&s_stage[0][0][0];
    const lds_ptr<uint8_t> tb = (lds_ptr<uint8_t>)&s_tiles;
    constexpr int kWT = (int)sizeof(WaveTiles);
    constexpr int oP = (int)offsetof(WaveTiles, P), oZ = (int)offsetof(WaveTiles, Z), oSV = (int)offsetof(WaveTiles, SV);
    const int rsel = 4 * G + (L16 >> 2), csel = 4 * (L16 & 3);
    const int o_vtr = w * kWT + 2 * (rsel * kSV + csel);       // V^T operand, + 32 per 16 channel positions
    const int o_vwr = w * kWT + 2 * (L16 * kSV + 16 * G);      // V row slice, + 128 per group
    const int o_ptr = w * kWT + oP + 2 * (rsel * kPS + csel);  // P^T operand
    const int o_pwr = w * kWT + oP + 2 * (L16 * kPS + 4 * G);
    const int o_ztr = w * kWT + oZ + 2 * (rsel * kPS + csel);
    const int o_zwr = w * kWT + oZ + 2 * (L16 * kPS);
    const int o_svr = w * kWT + oSV + 8 * G;                   // + 32 per group
    const int o_svw = w * kWT + oSV + 2 * L16;
    const int o_m = GE::SC + GE::SR + L16 * 4 * kGroups;        // + 4 per group
    const int o_c = L16 * (16 * GE::RS) + (BITS_C == 4 ? 8 : 4) * G;
    const int o_r = GE::SC + L16 * (kDr / 2) + 8 * G;

    // One pipelined step: PV of block t (tiles in LDS, probabilities pb) fused group by group with
    // QK of block t + 1 (staging zone (t + 1) % 3): group g's V-tile columns are read for block t
    // before block t + 1's codes overwrite them (a wave's LDS operations complete in order).  Block
    // t + 1 past the end gets scores -inf and leaves junk in the tiles that no PV reads.
    // Returns block t + 1's S (rows heads 4G + i, column token L16).
    auto step = [&](int t1, const f16x4 pb, const bool do_pv) -> f32x4 {
      const int zo = (w * kZones + t1 % kZones) * GE::SZ;
      // block t's zero and scale operands (the tiles are rewritten at the end of this step)
      f16x4 za = {}, sv[8];
      if (do_pv) {
        za = lds_tr4((lds_ptr<f16>)(tb + o_ztr));
#pragma unroll
        for (int g = 0; g < 8; ++g) sv[g] = lds_load<f16x4>(tb + (o_svr + 32 * g));
      }
      const int tok = (page0 + t1) * kPageTokens + row;
      const bool valid = t1 <= last && tok >= p_lo && tok < p_hi;
      uint32_t mw[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const uint32_t v = lds_load<uint32_t>(sb + (zo + o_m + 4 * g));
        mw[g] = valid ? v : 0u;
      }
      // (vector types: a struct load can be split into loads that lose their object)
      const u32x2 rw = lds_load<u32x2>(sb + (zo + o_r));
      // Per group: the LDS reads of group g + 1 are issued, then group g's codes are unpacked and
      // multiplied (the fences keep this order, so only two groups' operands are live), and each
      // group's partial is scaled into s one group later.
      // K operand words of block t + 1 (C4: units 2g, 2g + 1 of the token's row, the lane's 8 bytes
      // at 8 G; C2: unit g, the lane's dword at 4 G; group 8: the RoPE codes)
      auto rd_k = [&](int g) -> u32x2 {
        if (g == 8) return rw;
        if (BITS_C == 4) return lds_load<u32x2>(sb + (zo + o_c + 32 * g));
        return u32x2{lds_load<uint32_t>(sb + (zo + o_c + 16 * g)), 0u};
      };
      // V^T operands of block t, channel positions 64 g .. 64 g + 63
      auto rd_v = [&](int g, f16x4 (&va)[4]) {
        if (g < 8 && do_pv) {
#pragma unroll
          for (int c = 0; c < 4; ++c) va[c] = lds_tr4((lds_ptr<f16>)(tb + (o_vtr + 32 * (4 * g + c))));
        }
      };
      f32x4 s = {0.f, 0.f, 0.f, 0.f}, cprev;
      u32x2 kw_next = rd_k(0);
      f16x4 va_next[4];
      rd_v(0, va_next);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const u32x2 kw = kw_next;
        f16x4 va[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) va[c] = va_next[c];
        if (g + 1 < kGroups) {
          kw_next = rd_k(g + 1);
          rd_v(g + 1, va_next);
        }
        __builtin_amdgcn_sched_barrier(0);
        f16x8 k0, k1;
        if (g == 8 || BITS_C == 4) {
          k0 = __builtin_bit_cast(f16x8, unpack4(kw.x));
          k1 = __builtin_bit_cast(f16x8, unpack4(kw.y));
        } else {
          uint4 x0, x1;
          unpack2(kw.x, x0, x1);
          k0 = __builtin_bit_cast(f16x8, x0);
          k1 = __builtin_bit_cast(f16x8, x1);
        }
        f32x4 cg = mfma32k(qreg[2 * g], k0, f32x4{0.f, 0.f, 0.f, 0.f});
        cg = mfma32k(qreg[2 * g + 1], k1, cg);
        if (g < 8) {
          *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_vwr + 128 * g)) = k0;
          *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_vwr + 128 * g + 16)) = k1;
          if (do_pv) {
            const f16x4 bop = pb * sv[g];
#pragma unroll
            for (int c = 0; c < 4; ++c) O[4 * g + c] = mfma16k(va[c], bop, O[4 * g + c]);
          }
        }
        if (g > 0) s += bf16f(mw[g - 1] & 0xFFFFu) * cprev;
        cprev = cg;
        __builtin_amdgcn_sched_barrier(0);
      }
      s += bf16f(mw[kGroups - 1] & 0xFFFFu) * cprev;
      if (do_pv) oz = mfma16k(za, pb, oz);
      // block t + 1's Z and SV tile entries: lane (token L16, G) writes groups 2G, 2G + 1 (lanes G = 0
      // also z_8 into column 8; columns 9 .. 15 stay zero), then reads its zero-term operand back:
      // z_0 .. z_7 (G < 2) or z_8 and seven zeros (G >= 2)
      {
        const u32x2 mp = lds_load<u32x2>(sb + (zo + o_m + 8 * G));
        const uint32_t m0 = valid ? mp.x : 0u, m1 = valid ? mp.y : 0u;
        *reinterpret_cast<lds_ptr<f16x2>>(tb + (o_zwr + 4 * G)) = f16x2{(f16)bf16f(m0 >> 16), (f16)bf16f(m1 >> 16)};
        *reinterpret_cast<lds_ptr<f16>>(tb + (o_svw + 64 * G)) = (f16)bf16f(m0 & 0xFFFFu);
        *reinterpret_cast<lds_ptr<f16>>(tb + (o_svw + 64 * G + 32)) = (f16)bf16f(m1 & 0xFFFFu);
        if (G == 0) *reinterpret_cast<lds_ptr<f16>>(tb + (o_zwr + 16)) = (f16)bf16f(mw[8] >> 16);
      }
      const f16x8 zf = lds_load<f16x8>(tb + (o_zwr + 16 * (G >> 1)));
      s = mfma32k(qz, zf, s * c_log2) + (valid ? 0.f : -__builtin_inff());
      return s;
    };

    if (G == 0) *reinterpret_cast<lds_ptr<f16x8>>(tb + (o_zwr + 16)) = f16x8{};  // Z columns 8 .. 15
    // while block t's PV and block t + 1's QK run, blocks t + 2, t + 3 are in flight
    stage(0, page_id(0));
    stage(1, page_id(1));
    stage(2, page_id(2));
    int pg_next = page_id(3);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * GE::LOADS) : "memory");  // block 0 landed
    f32x4 S = step(0, f16x4{}, false);
    int t = 0;
    while (true) {
      if (needs_refresh(S)) refresh(S);  // rare: kept apart from the block loop
      while (t <= last) {
        stage(t + 3, pg_next);  // zone t % 3: block t's QK reads are done
        pg_next = page_id(t + 4);
        // softmax of block t, probabilities to LDS and back as the PV B operand (head L16)
        f16x4 pz;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float mu = m_run[i] == -__builtin_inff() ? 0.f : m_run[i];
          const float e = __builtin_amdgcn_exp2f(S[i] - mu);
          l_part[i] += e;
          pz[i] = (f16)e;
        }
        *reinterpret_cast<lds_ptr<f16x4>>(tb + o_pwr) = pz;
        const f16x4 pb = lds_tr4((lds_ptr<f16>)(tb + o_ptr));
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * GE::LOADS) : "memory");  // block t + 1 landed
        S = step(t + 1, pb, true);
        ++t;
        if (needs_refresh(S)) break;
      }
      if (t > last) break;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no staging left in flight
  } else {
    // bf16 tokens in virtual pages of 64, this wave's rows 16w .. 16w + 15 of each
    for (int t = 0; t < n_blocks; ++t) {
      const int j = t * kPageTokens + row;
      const bool valid = j < nb;
      const uint16_t* src = nullptr;  // masked lanes read nothing
      if (valid) {
        if (j < ns) src = p.sink + ((int64_t)slot * p.n_sink + j) * kD;
        else src = p.recent + ((int64_t)slot * p.n_recent + (rstart + (j - ns)) % p.n_recent) * kD;
      }
      float s_qk[kGroups], s_pv[kGroups], z[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        s_qk[g] = valid ? c_log2 : 0.f;
        s_pv[g] = valid ? 1.f : 0.f;
        z[g] = 0.f;
      }
      auto kv = [&](int g, int h) -> f16x8 {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (valid) raw = *reinterpret_cast<const uint4*>(src + 64 * g + 16 * G + 8 * h);
        return __builtin_bit_cast(f16x8, g < 8 ? bf16_chunk_to_f16<BITS_C>(raw) : bf16_chunk_to_f16<4>(raw));
      };
      const f32x4 S = block_qk(kv, s_qk, s_pv, z, valid ? 0.f : -__builtin_inff());
      if (needs_refresh(S)) refresh(S);
      softmax_pv(S);
    }
  }

  // ---- merge the four waves' partials (per head: max-shifted sums) and write the split's row
  __syncthreads();  // every wave is done with its tiles; the merge area overlays them
  auto& mg = s_tiles.mg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l_row = row16_sum(l_part[i]);
    if (L16 == 0) {
      mg.m[w][4 * G + i] = m_run[i];
      mg.l[w][4 * G + i] = l_row;
    }
  }
  __syncthreads();
  float M = -__builtin_inff();  // merged max of head L16 (the PV column)
#pragma unroll
  for (int v = 0; v < kW; ++v) M = fmaxf(M, mg.m[v][L16]);
  {
    const float mw = mg.m[w][L16];
    const float f = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) O[cb] *= f;
    oz *= f;
  }
  if (G < 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mg.z[w][L16][4 * G + i] = oz[i];
  }
  // waves 2, 3 hand their outputs to waves 0, 1; then wave 1 hands the sum to wave 0
  auto put = [&](int k) {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
      *reinterpret_cast<f32x4*>(&mg.o[k][L16][16 * cb + 4 * G]) = O[cb];
  };
  auto add = [&](int k) {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) O[cb] += *reinterpret_cast<const f32x4*>(&mg.o[k][L16][16 * cb + 4 * G]);
  };
  if (w >= 2) put(w - 2);
  __syncthreads();
  if (w < 2) add(w);
  __syncthreads();
  if (w == 1) put(0);
  __syncthreads();
  if (w == 0) {
    add(0);
    const int64_t orow = (int64_t)item * p.heads + head0 + L16;
    float* dst = p.ws_o + orow * kDc;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = 16 * cb + 4 * G + i;
        dst[8 * (pos >> 3) + perm8<BITS_C>(pos & 7)] = O[cb][i];
      }
    if (G == 0) {
      float L = 0.f, zs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kW; ++v) {
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

template <int BITS_C>
hipError_t launch16(const DecodeParams& p, hipStream_t stream) {
  const int64_t blocks = ((int64_t)p.max_items + 7) / 8 * 8 * p.head_groups;
  hipLaunchKernelGGL(decode16_kernel<BITS_C>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode16(const DecodeParams& p, int bits_c, hipStream_t stream) {
  if (bits_c == 4) return launch16<4>(p, stream);
  if (bits_c == 2) return launch16<2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
