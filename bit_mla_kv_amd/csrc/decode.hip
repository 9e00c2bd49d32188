// Split-KV low-bit MLA decode for gfx950 (CDNA4), plus the log-sum-exp combine.
//
// What is computed (QuantMLA pages: ai.info summary, "Key Contributions",
// item 4 and "Methodology in Plain English"; onedev.kr review, "How it is
// used"): for one query token per sequence and every head h,
//   sigma_t = scale * (q_c . c_t + q_r . k_r,t),  out_h = sum_t softmax(sigma)_t c_t
// over all N valid tokens, each token entering exactly once: tokens
// t < n_sink and t >= N - n_recent come from the bf16 sink / recent buffers,
// every other token from its packed copy, unpacked inside the loop.
//
// Work decomposition: one workgroup per (sequence, split, head group).
// Split 0 holds the bf16 tokens; splits 1.. hold page-aligned chunks of the
// packed range.  Each split leaves a normalised partial output and a log2
// log-sum-exp in the workspace; combine_kernel merges them exactly.
//
// Per 64-token tile the workgroup stages the page in an fp16 LDS tile:
// packed page bytes are prefetched into registers one tile ahead (128-bit
// loads) while the current tile computes, then unpacked to EXACT integer
// codes (nibbles / crumbs become fp8 bytes whose e4m3 value is code * 2^-9,
// converted with a 2^9 scale).  Each wave owns 16 query heads:
//   QK   per 64-channel group g:  acc_g = codes_g . q_g  (MFMA 16x16x32 f16, exact)
//        S += s'_g * acc_g        (fp32; s' = s * scale * log2 e)
//        zero terms: sum_g z_g * qsum_g through one extra MFMA step whose B
//        operand holds qsum split into fp16 hi + lo parts (RoPE group: fp32 FMA)
//   softmax in the log2 domain, running max refreshed lazily (only when it
//        grows by more than 2^8), probabilities kept in fp32 for the normaliser
//   PV   per group g: O_g += codes_g^T . fp16(p * s_g)   (MFMA; V^T operand read
//        with the gfx950 LDS transpose load ds_read_b64_tr_b16)
//        plus one MFMA block over the z columns with fp16(p) for sum_t p_t z_g,t.
// bf16 tiles use the same pipeline with s = 1 and z = 0.
#include <algorithm>
#include <cstdlib>

#include "decode_common.h"

namespace mla {
namespace {

using namespace dev;

constexpr int kTile = 64;        // tokens per tile (one page)
constexpr int kStride = 600;     // LDS tile row stride in halves (bank-spread for 16-row reads)
constexpr int kZPos = 576;       // z columns: [576,584) z_0..z_7, [584,592) z_0..z_7 again, [592,600) zero
constexpr float kRescale = 8.0f; // lazy max refresh threshold, log2 units

struct __align__(16) Smem {
  f16 tile[kTile * kStride + 16];  // +16: the z-column K step of the last row reads 8 halves past it
  float sq[kGroups][kTile];        // QK scale s * scale * log2(e); 0 for masked tokens
  float sv[8][kTile];              // PV scale s; 0 for masked tokens
  float zr[kTile];                 // RoPE-group zero; 0 for masked tokens
  float bias[kTile];               // 0 valid, -inf masked
};

// ---------------------------------------------------------------------------------------
// BITS_C: content code bits; HB: 16-head blocks per workgroup; TS: waves splitting a tile's tokens.
template <int BITS_C, int HB, int TS>
__global__ __launch_bounds__(64 * HB * TS) void decode_kernel(DecodeParams p) {
  constexpr int NT = 64 * HB * TS;
  constexpr int RT = kTile / TS;      // tokens per wave per tile
  constexpr int NBLK = RT / 16;       // 16-token MFMA blocks per wave per tile
  constexpr int CB = kDc * BITS_C / 8;
  constexpr int PB = kPageTokens * (CB + kDr / 2 + 4 * kGroups);
  constexpr int UC = kPageTokens * CB / 16;       // content chunks
  constexpr int UPR = CB / 16;                    // content chunks per token row
  constexpr int UR = kPageTokens * (kDr / 2) / 16;  // RoPE chunks (128)
  constexpr int CPT = UC / NT;                    // content chunks per thread
  constexpr int META_T0 = NT >= 256 ? 128 : 0;    // threads [META_T0, META_T0+64) own one token's metadata
  static_assert(UC % NT == 0 && UR == 128 && NT >= 128, "prefetch split assumes these sizes");
  static_assert(NBLK % 2 == 0, "PV consumes 32-token pairs of blocks");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hb = wave % HB;
  const int ts = wave / HB;
  const int G = lane >> 4;     // lane group (MFMA k slice)
  const int L16 = lane & 15;   // MFMA row/column within a 16 block

  // XCD-aware work mapping: blocks x and x + 8 run on the same XCD (round-robin dispatch over the
  // 8 XCDs), so the head groups of one (sequence, split) pair are consecutive blocks of one XCD
  // and share its L2 for the page stream.
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int hg = kx % p.head_groups;
  const int item = xcd + 8 * (kx / p.head_groups);
  if (item >= min(p.plan_hdr[0], p.max_items)) return;
  const int4 itm = reinterpret_cast<const int4*>(p.items)[item];
  const int b = itm.x;
  const int split = itm.w ? 0 : 1;  // 0: bf16 tokens, otherwise a packed chunk

  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  const int p_lo = p.n_sink;            // packed token range [p_lo, p_hi)
  const int p_hi = N - p.n_recent;
  const bool any_packed = p_hi > p_lo;
  const int first_page = p_lo / kPageTokens;
  const int n_pp = any_packed ? (p_hi - 1) / kPageTokens - first_page + 1 : 0;

  int n_iter;
  int page0 = 0;
  int ns = 0, nb = 0, rstart = 0;
  if (split == 0) {
    ns = min(p.n_sink, N);
    rstart = max(p.n_sink, N - p.n_recent);
    nb = ns + max(0, N - rstart);
    n_iter = (nb + kTile - 1) / kTile;
  } else {
    page0 = itm.y;
    n_iter = min(itm.z, first_page + n_pp - page0);
    if (n_iter <= 0) return;
  }

  const int head_base = hg * 16 * HB + hb * 16;
  const int my_head = head_base + L16;
  const float c_log2 = p.scale_log2e;

  // ---- queries: B operand of QK, positions ordered like the tile; 19 K steps of 32
  f16x8 qreg[19];
  float qs[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) qs[g] = 0.f;
  {
    const uint16_t* qh = p.q + ((int64_t)b * p.heads + my_head) * kD;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int cbase = 32 * ks + 8 * G;  // 8-channel block start (channel == position block)
      const uint4 raw = *reinterpret_cast<const uint4*>(qh + cbase);
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
    f16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16 hi = (f16)qs[j];
      const f16 lo = (f16)(qs[j] - (float)hi);
      z[j] = G == 0 ? hi : (G == 1 ? lo : (f16)0.f);
    }
    qreg[18] = z;
  }
  const float qr8 = qs[8];

  // ---- zero the never-written pad columns [592,600) and the slack once
  for (int r = tid; r < kTile; r += NT)
    *reinterpret_cast<uint4*>(&sm.tile[r * kStride + 592]) = make_uint4(0, 0, 0, 0);
  if (tid < 2) *reinterpret_cast<uint4*>(&sm.tile[kTile * kStride + 8 * tid]) = make_uint4(0, 0, 0, 0);

  // ---- per-lane state
  f32x4 O[33];
#pragma unroll
  for (int i = 0; i < 33; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_part = 0.f;

  // ---- packed prefetch registers (one page ahead): every thread has chunks of a fixed kind
  uint4 pfc[CPT];          // content codes: chunk tid + k*NT
  uint4 pfr;               // RoPE-key codes: chunk tid (tid < 128)
  uint32_t pfm[kGroups];   // metadata of token tid - META_T0
  const bool has_rope = tid < 128;
  const bool has_meta = tid >= META_T0 && tid < META_T0 + kPageTokens;
  const int64_t slot_row = (int64_t)slot * p.max_pages;
#define MLA_PREFETCH(page_idx)                                                                        \
  do {                                                                                                \
    const int pi_ = (page_idx);                                                                       \
    int64_t pg_ = (pi_ < p.max_pages) ? (int64_t)p.block_table[slot_row + pi_] : -1;                 \
    const bool ok_ = pg_ >= 0 && pg_ < p.num_pages;                                                   \
    const uint8_t* base_ = p.pages + (ok_ ? pg_ : 0) * (int64_t)PB;                                   \
    const u32x4* c_ = reinterpret_cast<const u32x4*>(base_);                                          \
    _Pragma("unroll") for (int k = 0; k < CPT; ++k) {                                                 \
      u32x4 v_ = {0u, 0u, 0u, 0u};                                                                    \
      if (ok_) v_ = __builtin_nontemporal_load(c_ + tid + k * NT);                                    \
      pfc[k] = make_uint4(v_[0], v_[1], v_[2], v_[3]);                                                \
    }                                                                                                 \
    if (has_rope) {                                                                                   \
      u32x4 v_ = {0u, 0u, 0u, 0u};                                                                    \
      if (ok_) v_ = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base_ + kPageTokens * CB) + tid); \
      pfr = make_uint4(v_[0], v_[1], v_[2], v_[3]);                                                   \
    }                                                                                                 \
    if (has_meta) {                                                                                   \
      const uint32_t* m_ = reinterpret_cast<const uint32_t*>(base_ + kPageTokens * (CB + kDr / 2)) +  \
                           (tid - META_T0) * kGroups;                                                 \
      _Pragma("unroll") for (int g = 0; g < kGroups; ++g) pfm[g] = ok_ ? __builtin_nontemporal_load(m_ + g) : 0u; \
    }                                                                                                 \
  } while (0)

  // ---- main loop
  __syncthreads();
  if (split != 0) MLA_PREFETCH(page0);
  for (int it = 0; it < n_iter; ++it) {
    __syncthreads();  // every wave is done reading the previous tile
    if (split == 0) {
      // bf16 sink / recent rows -> fp16 tile (same channel order as unpacked codes), s = 1, z = 0
      for (int e = tid; e < kTile * (kD / 8); e += NT) {
        const int r = e / (kD / 8), m = e % (kD / 8);
        const int j = it * kTile + r;
        uint4 o = make_uint4(0, 0, 0, 0);
        if (j < nb) {
          const uint16_t* src;
          if (j < ns) {
            src = p.sink + ((int64_t)slot * p.n_sink + j) * kD;
          } else {
            const int t = rstart + (j - ns);
            src = p.recent + ((int64_t)slot * p.n_recent + t % p.n_recent) * kD;
          }
          const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * m);
          o = m < kDc / 8 ? bf16_chunk_to_f16<BITS_C>(raw) : bf16_chunk_to_f16<4>(raw);
        }
        *reinterpret_cast<uint4*>(&sm.tile[r * kStride + 8 * m]) = o;
      }
      for (int r = tid; r < kTile; r += NT) {
        const bool valid = it * kTile + r < nb;
        for (int g = 0; g < kGroups; ++g) sm.sq[g][r] = valid ? c_log2 : 0.f;
        for (int g = 0; g < 8; ++g) sm.sv[g][r] = valid ? 1.f : 0.f;
        sm.zr[r] = 0.f;
        sm.bias[r] = valid ? 0.f : -__builtin_inff();
        *reinterpret_cast<uint4*>(&sm.tile[r * kStride + kZPos]) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&sm.tile[r * kStride + kZPos + 8]) = make_uint4(0, 0, 0, 0);
      }
    } else {
      // packed page (in registers) -> exact fp16 codes + per-token metadata in LDS
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int u = tid + k * NT;
        const uint4 v = pfc[k];
        const int r = u / UPR, ch = u % UPR;
        f16* dst = &sm.tile[r * kStride];
        if (BITS_C == 4) {
          *reinterpret_cast<uint4*>(dst + 32 * ch + 0) = unpack4(v.x);
          *reinterpret_cast<uint4*>(dst + 32 * ch + 8) = unpack4(v.y);
          *reinterpret_cast<uint4*>(dst + 32 * ch + 16) = unpack4(v.z);
          *reinterpret_cast<uint4*>(dst + 32 * ch + 24) = unpack4(v.w);
        } else {
          uint4 x0, x1;
          unpack2(v.x, x0, x1);
          *reinterpret_cast<uint4*>(dst + 64 * ch + 0) = x0;
          *reinterpret_cast<uint4*>(dst + 64 * ch + 8) = x1;
          unpack2(v.y, x0, x1);
          *reinterpret_cast<uint4*>(dst + 64 * ch + 16) = x0;
          *reinterpret_cast<uint4*>(dst + 64 * ch + 24) = x1;
          unpack2(v.z, x0, x1);
          *reinterpret_cast<uint4*>(dst + 64 * ch + 32) = x0;
          *reinterpret_cast<uint4*>(dst + 64 * ch + 40) = x1;
          unpack2(v.w, x0, x1);
          *reinterpret_cast<uint4*>(dst + 64 * ch + 48) = x0;
          *reinterpret_cast<uint4*>(dst + 64 * ch + 56) = x1;
        }
      }
      if (has_rope) {
        const int r = tid >> 1, half = tid & 1;
        f16* dst = &sm.tile[r * kStride + kDc + 32 * half];
        *reinterpret_cast<uint4*>(dst + 0) = unpack4(pfr.x);
        *reinterpret_cast<uint4*>(dst + 8) = unpack4(pfr.y);
        *reinterpret_cast<uint4*>(dst + 16) = unpack4(pfr.z);
        *reinterpret_cast<uint4*>(dst + 24) = unpack4(pfr.w);
      }
      if (has_meta) {
        const int r = tid - META_T0;
        const int t = (page0 + it) * kPageTokens + r;
        const bool valid = t >= p_lo && t < p_hi;
        f16 zh[8];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const float sc = valid ? bf16f(pfm[g] & 0xFFFFu) : 0.f;
          const float z = valid ? bf16f(pfm[g] >> 16) : 0.f;
          sm.sq[g][r] = sc * c_log2;
          if (g < 8) {
            sm.sv[g][r] = sc;
            zh[g] = (f16)z;
          } else {
            sm.zr[r] = z;
          }
        }
        uint4 zz;
        zz.x = __builtin_bit_cast(uint32_t, f16x2{zh[0], zh[1]});
        zz.y = __builtin_bit_cast(uint32_t, f16x2{zh[2], zh[3]});
        zz.z = __builtin_bit_cast(uint32_t, f16x2{zh[4], zh[5]});
        zz.w = __builtin_bit_cast(uint32_t, f16x2{zh[6], zh[7]});
        *reinterpret_cast<uint4*>(&sm.tile[r * kStride + kZPos]) = zz;
        *reinterpret_cast<uint4*>(&sm.tile[r * kStride + kZPos + 8]) = zz;
        sm.bias[r] = valid ? 0.f : -__builtin_inff();
      }
    }
    __syncthreads();
    if (split != 0 && it + 1 < n_iter) MLA_PREFETCH(page0 + it + 1);

    const int row0 = ts * RT;
    f32x4 S[NBLK];
    // -- QK: exact codes x fp16 q per group, fp32 group scale, zero terms
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk) {
      const int rb = row0 + 16 * bk;
      const f16* arow = &sm.tile[(rb + L16) * kStride + 8 * G];
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma(lds_read8(arow + 64 * g), qreg[2 * g], acc);
        acc = mfma(lds_read8(arow + 64 * g + 32), qreg[2 * g + 1], acc);
        const f32x4 sc = *reinterpret_cast<const f32x4*>(&sm.sq[g][rb + 4 * G]);
        sacc += sc * acc;
        __builtin_amdgcn_sched_barrier(0);
      }
      f32x4 accz = {0.f, 0.f, 0.f, 0.f};
      accz = mfma(lds_read8(arow + kZPos), qreg[18], accz);
      const f32x4 zr = *reinterpret_cast<const f32x4*>(&sm.zr[rb + 4 * G]);
      const f32x4 bias = *reinterpret_cast<const f32x4*>(&sm.bias[rb + 4 * G]);
      S[bk] = sacc + accz + zr * qr8 + bias;
      __builtin_amdgcn_sched_barrier(0);
    }
    // -- online softmax (log2 domain), lazy max refresh
    float mx = fmax4(S[0]);
#pragma unroll
    for (int bk = 1; bk < NBLK; ++bk) mx = fmaxf(mx, fmax4(S[bk]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescale)) {
      const float m_new = fmaxf(m_run, mx);
      // m_run = -inf (nothing seen yet) gives alpha = 0; m_new = -inf leaves the state alone
      const float alpha = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < 33; ++i) O[i] *= alpha;
    }
    const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[bk][i] = __builtin_amdgcn_exp2f(S[bk][i] - m_use);
      l_part += (S[bk][0] + S[bk][1]) + (S[bk][2] + S[bk][3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // -- PV over 32-token pairs of blocks; V^T operand through the LDS transpose load
#pragma unroll
    for (int pr = 0; pr < NBLK / 2; ++pr) {
      const int rb0 = row0 + 32 * pr, rb1 = rb0 + 16;
      const f32x4 p0 = S[2 * pr], p1 = S[2 * pr + 1];
      const f16* a0 = &sm.tile[(rb0 + 4 * G + (L16 >> 2)) * kStride + 4 * (L16 & 3)];
      const f16* a1 = &sm.tile[(rb1 + 4 * G + (L16 >> 2)) * kStride + 4 * (L16 & 3)];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(&sm.sv[g][rb0 + 4 * G]);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sm.sv[g][rb1 + 4 * G]);
        const f32x4 q0 = p0 * s0, q1 = p1 * s1;
        f16x8 bop;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bop[i] = (f16)q0[i];
          bop[4 + i] = (f16)q1[i];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int cb = 4 * g + c;
          const f16x4 lo = lds_tr4(a0 + 16 * cb), hi = lds_tr4(a1 + 16 * cb);
          const f16x8 aop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          O[cb] = mfma(aop, bop, O[cb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      f16x8 bz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bz[i] = (f16)p0[i];
        bz[4 + i] = (f16)p1[i];
      }
      const f16x4 lo = lds_tr4(a0 + kZPos), hi = lds_tr4(a1 + kZPos);
      const f16x8 aop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      O[32] = mfma(aop, bz, O[32]);
    }
  }
#undef MLA_PREFETCH

  // ---- finalise: full normaliser, fold zero-term block into content blocks
  float l_tot = l_part;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const float zs = __shfl(O[32][g & 3], L16 + 16 * (g >> 2), 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) O[4 * g + c] += zs;
  }

  float M = m_run;
  if (TS > 1) {
    __syncthreads();  // tile no longer read
    float* scratch = reinterpret_cast<float*>(sm.tile);
    float* ml = scratch + (TS - 1) * HB * 32 * 4 * 64;  // [TS][HB][16][2]
    if (G == 0) {
      ml[((ts * HB + hb) * 16 + L16) * 2 + 0] = m_run;
      ml[((ts * HB + hb) * 16 + L16) * 2 + 1] = l_tot;
    }
    __syncthreads();
    M = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < TS; ++t) M = fmaxf(M, ml[((t * HB + hb) * 16 + L16) * 2]);
    const float f = (M == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
    for (int i = 0; i < 32; ++i) O[i] *= f;
    if (ts > 0) {
      float* dst = scratch + ((ts - 1) * HB + hb) * 32 * 4 * 64;
#pragma unroll
      for (int i = 0; i < 32; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(i * 4 + j) * 64 + lane] = O[i][j];
    }
    __syncthreads();
    if (ts > 0) return;
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < TS; ++t) {
      const float mt = ml[((t * HB + hb) * 16 + L16) * 2];
      const float lt = ml[((t * HB + hb) * 16 + L16) * 2 + 1];
      lsum += (M == -__builtin_inff()) ? 0.f : lt * __builtin_amdgcn_exp2f(mt - M);
    }
    l_tot = lsum;
#pragma unroll
    for (int t = 1; t < TS; ++t) {
      const float* src = scratch + ((t - 1) * HB + hb) * 32 * 4 * 64;
#pragma unroll
      for (int i = 0; i < 32; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) O[i][j] += src[(i * 4 + j) * 64 + lane];
    }
  }

  // ---- write the unnormalised partial with its running max and sum
  const int64_t row = (int64_t)item * p.heads + my_head;
  float* dst = p.ws_o + row * kDc;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = 16 * cb + 4 * G + i;
      dst[8 * (pos >> 3) + perm8<BITS_C>(pos & 7)] = O[cb][i];
    }
  if (G == 0) {
    p.ws_ml[2 * row] = M;
    p.ws_ml[2 * row + 1] = l_tot;
  }
}

template <int BITS_C, int HB, int TS>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const size_t smem = sizeof(Smem);
  auto kern = decode_kernel<BITS_C, HB, TS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int64_t blocks = ((int64_t)p.max_items + 7) / 8 * 8 * p.head_groups;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * HB * TS), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

bool decode_config(int heads, int n_sink, int n_recent, int batch, int max_seq_len, DecodeConfig* cfg) {
  (void)n_sink;
  if (heads == 16) {
    cfg->heads_per_wg = 16; cfg->threads = 128; cfg->wg_per_cu = 2;
  } else if (heads == 32) {
    cfg->heads_per_wg = 32; cfg->threads = 256; cfg->wg_per_cu = 1;
  } else if (heads > 0 && heads % 64 == 0) {
    cfg->heads_per_wg = 64; cfg->threads = 512; cfg->wg_per_cu = 1;
  } else {
    return false;
  }
  int num_cu = 256;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) num_cu = v;
  }
  const int64_t head_groups = heads / cfg->heads_per_wg;
  int64_t target = std::max<int64_t>(1, (int64_t)num_cu * cfg->wg_per_cu / head_groups);
  if (const char* env = getenv("MLA_LOWBIT_TARGET_ITEMS")) {
    const long v = strtol(env, nullptr, 10);
    if (v > 0) target = v;
  }
  cfg->target_items = (int)std::min<int64_t>(target, 1 << 20);
  cfg->min_pages_per_split = 4;
  cfg->force_pages_per_split = 0;
  if (const char* env = getenv("MLA_LOWBIT_PAGES_PER_SPLIT")) {
    const long v = strtol(env, nullptr, 10);
    if (v > 0) cfg->force_pages_per_split = (int)std::min<long>(v, 1 << 20);
  }
  const int64_t max_pp = std::max<int64_t>(0, ((int64_t)max_seq_len - n_recent + kPageTokens - 1) / kPageTokens);
  int64_t packed_items;
  if (cfg->force_pages_per_split > 0)
    packed_items = (int64_t)batch * ((max_pp + cfg->force_pages_per_split - 1) / cfg->force_pages_per_split);
  else  // full chunks <= total / chunk <= target, plus at most one tail chunk per sequence
    packed_items = std::min<int64_t>((int64_t)batch * ((max_pp + cfg->min_pages_per_split - 1) / cfg->min_pages_per_split),
                                     cfg->target_items + (int64_t)batch);
  cfg->max_items = (int)std::min<int64_t>(packed_items + batch, 1 << 30);
  return true;
}

hipError_t launch_decode(const DecodeParams& p, int bits_c, hipStream_t stream) {
  const int hpw = p.heads / p.head_groups;
  if (hpw == 64) return launch_decode64(p, bits_c, stream);
  if (bits_c == 4) {
    if (hpw == 16) return launch_t<4, 1, 2>(p, stream);
    if (hpw == 32) return launch_t<4, 2, 2>(p, stream);
    if (hpw == 64) return launch_t<4, 4, 1>(p, stream);
  } else if (bits_c == 2) {
    if (hpw == 16) return launch_t<2, 1, 2>(p, stream);
    if (hpw == 32) return launch_t<2, 2, 2>(p, stream);
    if (hpw == 64) return launch_t<2, 4, 1>(p, stream);
  }
  return hipErrorInvalidValue;
}


}  // namespace mla
