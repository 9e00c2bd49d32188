// Split-KV low-bit MLA decode for 128-head groups on gfx950 (CDNA4).
//
// Same computation as decode.hip (QuantMLA pages: ai.info summary, "Key
// Contributions", item 4; onedev.kr review, "How it is used"): one global
// softmax over all valid tokens, sink / recent tokens from bf16, all others
// from their packed copies, output aggregated over the content latent.
//
// Work layout for 128 heads sharing one latent (one workgroup, 8 waves, one
// (sequence, split, 128-head group)):
//  - packed pages land in an LDS staging buffer straight from HBM
//    (global_load_lds_dwordx4, one page ahead); the workgroup unpacks them
//    once into an fp16 tile of exact codes plus per-token scales;
//  - QK is split by heads: wave w scores its 16 heads (MFMA 16x16x32 f16 on
//    exact codes, fp32 group scales, zero terms), runs the online softmax
//    (lazily refreshed max) and publishes fp16 probabilities, its rescale
//    factors and the zero-term aggregate sum_t p_t z_t,g (one more MFMA);
//  - PV is split by channels: wave w owns content group w for all 128 heads
//    (MFMA 32x32x16 f16): B = p * s_w built with packed fp16 multiplies from
//    the shared probabilities, A = V^T from the LDS transpose load, so every
//    V element is read from LDS exactly once per workgroup.
// Partials are left unnormalised with their running max and sum; the combine
// kernel adds the zero terms and merges splits.
#include <algorithm>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kT = 64;              // tokens per tile (one page)
constexpr int kS = 584;             // LDS row stride in halves: 292 dwords, conflict-free 16-row b128 reads
constexpr int kZ = 576;             // z columns [576, 584)
constexpr int kPS = 36;             // probability row stride (halves): conflict-free 8-byte column reads
constexpr float kRescale = 8.0f;    // lazy max refresh threshold, log2 units

template <int BITS_C>
struct Geo {
  static constexpr int CB = kDc * BITS_C / 8;                    // content bytes per token
  static constexpr int PB = kPageTokens * (CB + kDr / 2 + 4 * kGroups);
  static constexpr int UCH = PB / 16;                            // 16-byte chunks per page
  static constexpr int UC = kPageTokens * CB / 16;               // content chunks
  static constexpr int CDW = kPageTokens * CB / 4;               // content dwords
  static constexpr int DPR = CB / 4;                             // content dwords per token row
  static constexpr int META = kPageTokens * (CB + kDr / 2);      // metadata byte offset
};

template <int BITS_C>
struct __align__(16) Smem128 {
  f16 tile[kT * kS + 32];      // +32: zero-term V^T reads of row 63 run past the tile
  f16 svh[8][kT];              // PV group scale s (fp16); 0 for masked tokens
  float sq[kGroups][kT];       // QK group scale s * scale * log2 e; 0 for masked tokens
  float zr[kT];                // RoPE-group zero; 0 for masked tokens
  float bias[kT];              // 0 valid, -inf masked
  f16 prob[2][128][kPS];       // fp16 probabilities of the current 32-token half tile (double buffered)
  float alpha[2][128];         // per-head rescale factor for the PV accumulators
  int resc[2][8];              // per-wave "some head rescaled" flags
  f16x8 qfrag[3][8][64];       // per wave, per lane: QK B fragments of the RoPE K steps and the zero-term step
  uint8_t stage[Geo<BITS_C>::PB];  // packed page landing zone
  uint8_t guard[1024];             // keeps a full wave's 1 KB landing window inside the allocation
};

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}


template <int BITS_C>
__global__ __launch_bounds__(512) void decode128_kernel(DecodeParams p) {
  using GE = Geo<BITS_C>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem128<BITS_C>& sm = *reinterpret_cast<Smem128<BITS_C>*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;        // wave: QK heads [16w, 16w+16), PV content group w
  const int G = lane >> 4;       // 16x16x32 k slice
  const int L16 = lane & 15;
  const int half = lane >> 5;    // 32x32x16 k half
  const int l32 = lane & 31;

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
  const int p_lo = p.n_sink, p_hi = N - p.n_recent;
  const int first_page = p_lo / kPageTokens;
  const int n_pp = p_hi > p_lo ? (p_hi - 1) / kPageTokens - first_page + 1 : 0;
  int n_iter, page0 = 0, ns = 0, nb = 0, rstart = 0;
  if (split == 0) {
    ns = min(p.n_sink, N);
    rstart = max(p.n_sink, N - p.n_recent);
    nb = ns + max(0, N - rstart);
    n_iter = (nb + kT - 1) / kT;
  } else {
    page0 = itm.y;
    n_iter = min(itm.z, first_page + n_pp - page0);
    if (n_iter <= 0) return;
  }

  const int head0 = hg * 128;
  const int qk_head = head0 + 16 * w + L16;  // head scored by this lane
  const float c_log2 = p.scale_log2e;

  // ---- queries: B operand of QK 16x16x32 (lane: head qk_head, positions 32 ks + 8 G + j)
  f16x8 qreg[16];   // content K steps; RoPE steps and the zero-term step live in LDS (qfrag)
  float qr8;
  {
    float qs[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) qs[g] = 0.f;
    const uint16_t* qh = p.q + ((int64_t)b * p.heads + qk_head) * kD;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qh + 32 * ks + 8 * G);
      const uint4 hv = ks < 16 ? bf16_chunk_to_f16<BITS_C>(raw) : bf16_chunk_to_f16<4>(raw);
      const f16x8 fr = __builtin_bit_cast(f16x8, hv);
      if (ks < 16) qreg[ks] = fr;
      else sm.qfrag[ks - 16][w][lane] = fr;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += (float)fr[j];
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
    sm.qfrag[2][w][lane] = z;
    qr8 = qs[8];
  }

  if (tid < 4) *reinterpret_cast<uint4*>(&sm.tile[kT * kS + 8 * tid]) = make_uint4(0, 0, 0, 0);

  // ---- state: QK role (softmax of own heads, zero-term aggregate), PV role (channels of group w)
  float m_run = -__builtin_inff();
  float l_part = 0.f;
  f32x4 oz = {0.f, 0.f, 0.f, 0.f};   // rows 576 + 4G + i: sum_t p z_(4G+i) for head qk_head (G < 2)
  f32x16 O[4][2];                    // [head block][channel block] of group w
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) O[hb][0] = O[hb][1] = f32x16{};

  const int64_t slot_row = (int64_t)slot * p.max_pages;
  auto prefetch = [&](int page_idx) {
    const int64_t pg = (page_idx < p.max_pages) ? (int64_t)p.block_table[slot_row + page_idx] : -1;
    if (pg < 0 || pg >= p.num_pages) return;  // contract violation: stale staging data, no fault
    const uint8_t* src = p.pages + pg * (int64_t)GE::PB;
#pragma unroll
    for (int r = 0; r < (GE::UCH + 511) / 512; ++r) {
      const int c0 = r * 512 + w * 64;  // wave-uniform first chunk
      if (c0 < GE::UCH && c0 + lane < GE::UCH)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(src + (int64_t)(c0 + lane) * 16),
            reinterpret_cast<__attribute__((address_space(3))) void*>(
                reinterpret_cast<uintptr_t>(sm.stage + c0 * 16)), 16, 0, 0);
    }
  };

  __syncthreads();
  if (split != 0) prefetch(page0);

  for (int it = 0; it < n_iter; ++it) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // staging landed for every wave; previous tile fully consumed
    if (split == 0) {
      for (int e = tid; e < kT * (kD / 8); e += 512) {
        const int r = e / (kD / 8), m = e % (kD / 8);
        const int j = it * kT + r;
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
        *reinterpret_cast<uint4*>(&sm.tile[r * kS + 8 * m]) = o;
      }
      if (tid < kT) {
        const int r = tid;
        const bool valid = it * kT + r < nb;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) sm.sq[g][r] = valid ? c_log2 : 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) sm.svh[g][r] = valid ? (f16)1.f : (f16)0.f;
        sm.zr[r] = 0.f;
        sm.bias[r] = valid ? 0.f : -__builtin_inff();
        *reinterpret_cast<uint4*>(&sm.tile[r * kS + kZ]) = make_uint4(0, 0, 0, 0);
      }
    } else {
      // content codes, one packed dword per lane and step: consecutive lanes write consecutive
      // 16-byte (C4) or 32-byte (C2) runs of the tile, which keeps the LDS writes conflict-free
#pragma unroll 4
      for (int k = 0; k < GE::CDW / 512; ++k) {
        const int u = tid + k * 512;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(sm.stage + 4 * u);
        const int r = u / GE::DPR, d = u % GE::DPR;
        f16* dst = &sm.tile[r * kS];
        if (BITS_C == 4) {
          *reinterpret_cast<uint4*>(dst + 8 * d) = unpack4(v);
        } else {
          uint4 x0, x1;
          unpack2(v, x0, x1);
          *reinterpret_cast<uint4*>(dst + 16 * d) = x0;
          *reinterpret_cast<uint4*>(dst + 16 * d + 8) = x1;
        }
      }
      if (tid < 128) {  // RoPE-key codes: token tid/2, channels 32*(tid&1) .. +31
        const uint4 v = *reinterpret_cast<const uint4*>(sm.stage + 16 * (GE::UC + tid));
        f16* dst = &sm.tile[(tid >> 1) * kS + kDc + 32 * (tid & 1)];
        *reinterpret_cast<uint4*>(dst + 0) = unpack4(v.x);
        *reinterpret_cast<uint4*>(dst + 8) = unpack4(v.y);
        *reinterpret_cast<uint4*>(dst + 16) = unpack4(v.z);
        *reinterpret_cast<uint4*>(dst + 24) = unpack4(v.w);
      } else if (tid < 128 + kT) {  // metadata of token tid - 128
        const int r = tid - 128;
        const uint32_t* md = reinterpret_cast<const uint32_t*>(sm.stage + GE::META) + r * kGroups;
        const int t = (page0 + it) * kPageTokens + r;
        const bool valid = t >= p_lo && t < p_hi;
        f16 zh[8];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const uint32_t wd = md[g];
          const float sc = valid ? bf16f(wd & 0xFFFFu) : 0.f;
          const float z = valid ? bf16f(wd >> 16) : 0.f;
          sm.sq[g][r] = sc * c_log2;
          if (g < 8) {
            sm.svh[g][r] = (f16)sc;
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
        *reinterpret_cast<uint4*>(&sm.tile[r * kS + kZ]) = zz;
        sm.bias[r] = valid ? 0.f : -__builtin_inff();
      }
    }
    __syncthreads();
    if (split != 0 && it + 1 < n_iter) prefetch(page0 + it + 1);

#pragma unroll 1
    for (int sub = 0; sub < 2; ++sub) {
      const int r0 = 32 * sub;
      const int par = sub;  // two half tiles per page: parity = sub
      const lds_ptr<f16> tb = lds_opaque(sm.tile);
      // ===== QK role: 16 heads x 32 tokens (two 16-token blocks)
      f32x4 S[2];
      {
        const lds_ptr<float> sq = lds_opaque(&sm.sq[0][0]);
        const lds_ptr<float> zp = lds_opaque(&sm.zr[0]);
        const lds_ptr<float> bp = lds_opaque(&sm.bias[0]);
        const lds_ptr<f16x8> qf = lds_opaque(&sm.qfrag[0][w][lane]);
        // the two 16-token blocks form two independent MFMA chains per group
        const lds_ptr<f16> arow0 = tb + (r0 + L16) * kS + 8 * G;
        const lds_ptr<f16> arow1 = arow0 + 16 * kS;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const f16x8 q0 = g < 8 ? qreg[2 * g] : lds_load<f16x8>(qf);
          const f16x8 q1 = g < 8 ? qreg[2 * g + 1] : lds_load<f16x8>(qf + 8 * 64);
          const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
          f32x4 c0 = mfma16(lds_load<f16x8>(arow0 + 64 * g), q0, z4);
          f32x4 c1 = mfma16(lds_load<f16x8>(arow1 + 64 * g), q0, z4);
          c0 = mfma16(lds_load<f16x8>(arow0 + 64 * g + 32), q1, c0);
          c1 = mfma16(lds_load<f16x8>(arow1 + 64 * g + 32), q1, c1);
          const f32x4 sc0 = lds_load<f32x4>(sq + g * kT + r0 + 4 * G);
          const f32x4 sc1 = lds_load<f32x4>(sq + g * kT + r0 + 16 + 4 * G);
          s0 += sc0 * c0;
          s1 += sc1 * c1;
        }
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
          // zero terms of the content groups: every lane reads z_0..z_7 (B: hi / lo parts of qsum)
          const lds_ptr<f16> zrow = tb + (r0 + 16 * bk + L16) * kS + kZ;
          const f32x4 accz = mfma16(lds_load<f16x8>(zrow), lds_load<f16x8>(qf + 16 * 64), f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 zv = lds_load<f32x4>(zp + r0 + 16 * bk + 4 * G);
          const f32x4 bv = lds_load<f32x4>(bp + r0 + 16 * bk + 4 * G);
          S[bk] = (bk == 0 ? s0 : s1) + accz + zv * qr8 + bv;
        }
      }
      // online softmax for the 16 heads (log2 domain, lazy max refresh)
      float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                       fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool need = mx > m_run + kRescale;
      float alpha = 1.f;
      if (need) {
        const float m_new = fmaxf(m_run, mx);
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // m_run = -inf -> 0
        m_run = m_new;
        l_part *= alpha;
        oz *= alpha;
      }
      const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[bk][i] = __builtin_amdgcn_exp2f(S[bk][i] - m_use);
        l_part += (S[bk][0] + S[bk][1]) + (S[bk][2] + S[bk][3]);
      }
      f16x8 pz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pz[i] = (f16)S[0][i];
        pz[4 + i] = (f16)S[1][i];
      }
      {
        // zero-term aggregate: rows z_0..z_7 of the tile's z columns (k: tokens 4G+j | 16+4G+j)
        const lds_ptr<f16> za = tb + (r0 + 4 * G + (L16 >> 2)) * kS + kZ + 4 * (L16 & 3);
        const f16x4 lo = lds_tr4(za), hi = lds_tr4(za + 16 * kS);
        const f16x8 aop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oz = mfma16(aop, pz, oz);
      }
      // publish probabilities (fp16) and the rescale factor of each head
      {
        f16* prow = &sm.prob[par][16 * w + L16][0];
        *reinterpret_cast<f16x4*>(prow + 4 * G) = f16x4{pz[0], pz[1], pz[2], pz[3]};
        *reinterpret_cast<f16x4*>(prow + 16 + 4 * G) = f16x4{pz[4], pz[5], pz[6], pz[7]};
        if (G == 0) sm.alpha[par][16 * w + L16] = alpha;
        const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
        if (lane == 0) sm.resc[par][w] = any ? 1 : 0;
      }
      __syncthreads();
      // ===== PV role: channels of group w (positions [64w, 64w+64)), all 128 heads
      {
        const lds_ptr<int> rf = lds_opaque(&sm.resc[par][0]);
        int anyr = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) anyr |= rf[k];
        if (anyr) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const float a = sm.alpha[par][32 * hb + l32];
            O[hb][0] *= a;
            O[hb][1] *= a;
          }
        }
        const lds_ptr<f16> svw = lds_opaque(&sm.svh[w][0]);
        const lds_ptr<f16> pr = lds_opaque(&sm.prob[par][0][0]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int t0 = 16 * ks + 4 * half;  // k slots: tokens t0 + j (j < 4), t0 + 8 + (j - 4)
          const f16x4 s0 = lds_load<f16x4>(svw + r0 + t0);
          const f16x4 s1 = lds_load<f16x4>(svw + r0 + t0 + 8);
          const f16x8 sv8 = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
          const lds_ptr<f16> va = tb + (r0 + t0 + ((lane & 15) >> 2)) * kS + 64 * w + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          f16x8 aop[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const f16x4 lo = lds_tr4(va + 32 * c), hi = lds_tr4(va + 8 * kS + 32 * c);
            aop[c] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const lds_ptr<f16> prow = pr + (32 * hb + l32) * kPS + t0;
            const f16x4 p0 = lds_load<f16x4>(prow);
            const f16x4 p1 = lds_load<f16x4>(prow + 8);
            const f16x8 pv = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            const f16x8 bop = pv * sv8;
            O[hb][0] = mfma32(aop[0], bop, O[hb][0]);
            O[hb][1] = mfma32(aop[1], bop, O[hb][1]);
          }
        }
      }
    }
  }

  // ---- unnormalised partial: O (PV role), running max / sum and zero-term sums (QK role)
  const int64_t rows = item;
  float* dst_o = p.ws_o + rows * p.heads * kDc;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    float* dh = dst_o + (int64_t)(head0 + 32 * hb + l32) * kDc;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = 64 * w + 32 * c + 8 * (i >> 2) + 4 * half + (i & 3);
        dh[8 * (pos >> 3) + perm8<BITS_C>(pos & 7)] = O[hb][c][i];
      }
  }
  float l_tot = l_part;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int64_t hrow = rows * p.heads + qk_head;
  if (G == 0) {
    p.ws_ml[2 * hrow] = m_run;
    p.ws_ml[2 * hrow + 1] = l_tot;
  }
  if (G < 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p.ws_z[hrow * 8 + 4 * G + i] = oz[i];
  }
}

template <int BITS_C>
hipError_t launch128(const DecodeParams& p, hipStream_t stream) {
  const size_t smem = sizeof(Smem128<BITS_C>);
  auto kern = decode128_kernel<BITS_C>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int64_t blocks = ((int64_t)p.max_items + 7) / 8 * 8 * p.head_groups;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(512), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode128(const DecodeParams& p, int bits_c, hipStream_t stream) {
  if (bits_c == 4) return launch128<4>(p, stream);
  if (bits_c == 2) return launch128<2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
