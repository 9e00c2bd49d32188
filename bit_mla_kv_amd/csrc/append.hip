// Fused quantize-append writer for the low-bit MLA cache (gfx950).
//
// One wavefront per new token, one lane per channel of each 64-channel group.
// Per group: wave-wide min/max, scale s = bf16(fp32(max - min) / (2^b - 1)),
// zero z = min, codes rint_half_even(fp32(x - min) / s) clamped to [0, 2^b-1]
// (per-token asymmetric affine quantizer, group size 64: ai.info summary,
// "Methodology in Plain English"; onedev.kr review, "Premises and limits").
// Codes are OR-reduced across lanes into packed dwords and stored with the
// group's metadata dword into the token's page row; the bf16 row is copied to
// the sink buffer (first n_sink positions) and to the recent ring (last
// n_recent positions of the slot after this call), which is the whole of the
// migration rule: a token that leaves the window is served from the packed
// copy written here (onedev.kr review, "How it is used").
//
// Built with -ffp-contract=off; the arithmetic has no a*b+c anyway.
#include "mla_internal.h"

namespace mla {
namespace {

__device__ __forceinline__ float bf16_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Cross-lane reductions with DPP row operations (plain VALU instructions; a ds_bpermute shuffle
// costs an LDS round trip and each group's quantizer is a chain of such steps).  A lane whose DPP
// source lies outside its 16-lane row, or in a row outside the row mask, takes the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float x, float identity) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

// OR over each aligned group of W (8 or 16) consecutive lanes, complete in the group's first lane:
// lane i ORs lanes i + 1, i + 2, i + 4 (, i + 8) of its row (row_shl)
template <int W>
__device__ __forceinline__ uint32_t or_reduce(uint32_t v) {
  v |= dpp_u<0x101, 0xf>(v, 0u);
  v |= dpp_u<0x102, 0xf>(v, 0u);
  v |= dpp_u<0x104, 0xf>(v, 0u);
  if (W == 16) v |= dpp_u<0x108, 0xf>(v, 0u);
  return v;
}

// min / max over the 64 lanes (every lane gets the result): an inclusive scan in lane order (row
// shifts by 1, 2, 4, 8, then row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3),
// whose last lane holds the whole
template <typename Op>
__device__ __forceinline__ float wave_scan_last(float x, float identity, Op op) {
  x = op(x, dpp_f<0x111, 0xf>(x, identity));
  x = op(x, dpp_f<0x112, 0xf>(x, identity));
  x = op(x, dpp_f<0x114, 0xf>(x, identity));
  x = op(x, dpp_f<0x118, 0xf>(x, identity));
  x = op(x, dpp_f<0x142, 0xa>(x, identity));
  x = op(x, dpp_f<0x143, 0xc>(x, identity));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_min(float v) {
  return wave_scan_last(v, __builtin_inff(), [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_scan_last(v, -__builtin_inff(), [](float a, float b) { return fmaxf(a, b); });
}

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= p.n_tokens) return;
  const int slot = p.token_slot[tok];
  const int pos = p.token_pos[tok];
  if (slot < 0 || slot >= p.num_slots || pos < 0) return;
  const uint16_t* row = p.kv + (int64_t)tok * kD;
  // every load of the token's row is requested before any is used: the lane's channel of each
  // group, and the row's 16-byte chunks lane, 64 + lane for the bf16 copies
  float xs[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) xs[g] = bf16_to_float(row[g * kGroup + lane]);
  const uint4* src = reinterpret_cast<const uint4*>(row);
  const uint4 chunk0 = src[lane];
  const uint4 chunk1 = lane < kD / 8 - 64 ? src[64 + lane] : make_uint4(0, 0, 0, 0);

  // page row of this token (skip packed write if the table entry is out of range)
  uint8_t* prow_c = nullptr;
  uint8_t* prow_r = nullptr;
  uint32_t* prow_m = nullptr;
  const int pidx = pos / kPageTokens;
  if (pidx < p.max_pages) {
    const int64_t page = p.block_table[(int64_t)slot * p.max_pages + pidx];
    if (page >= 0 && page < p.num_pages) {
      const int r = pos % kPageTokens;
      const int cb = content_row_bytes(p.bits_c);
      uint8_t* base = p.pages + page * (int64_t)page_bytes(p.bits_c);
      prow_c = base + r * cb;
      prow_r = base + kPageTokens * cb + r * (kDr / 2);
      prow_m = reinterpret_cast<uint32_t*>(base + kPageTokens * (cb + kDr / 2)) + r * kGroups;
    }
  }

  if (prow_c) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int bits = g < 8 ? p.bits_c : 4;
      const int lb = (1 << bits) - 1;
      const float x = xs[g];
      const float mn = wave_min(x);
      const float mx = wave_max(x);
      const float range = mx - mn;
      const float s32 = __fdiv_rn(range, (float)lb);
      uint16_t sb = float_to_bf16_rne(s32);
      if ((sb & 0x7FFFu) == 0) sb = 0;  // a zero scale is stored as +0
      const float s = bf16_to_float(sb);
      uint16_t zb = float_to_bf16_rne(mn);  // exact: mn is a bf16 value
      if (zb == 0x8000u) zb = 0;             // -0 stored as +0
      uint32_t code = 0;
      if (s != 0.0f) {
        float d = __builtin_rintf(__fdiv_rn(x - mn, s));
        d = fminf(fmaxf(d, 0.0f), (float)lb);
        code = (uint32_t)d;
      }
      if (bits == 4) {
        const uint32_t w = or_reduce<8>(code << (4 * (lane & 7)));
        if ((lane & 7) == 0) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(g < 8 ? prow_c : prow_r);
          dst[((g < 8 ? g : 0) * kGroup + lane) / 8] = w;
        }
      } else {  // 2-bit content
        const uint32_t w = or_reduce<16>(code << (2 * (lane & 15)));
        if ((lane & 15) == 0) reinterpret_cast<uint32_t*>(prow_c)[(g * kGroup + lane) / 16] = w;
      }
      if (lane == 0) prow_m[g] = (uint32_t)sb | ((uint32_t)zb << 16);
    }
  }

  // bf16 copies: 1152 bytes = 72 x 16 bytes per row
  if (pos < p.n_sink) {
    uint4* dst = reinterpret_cast<uint4*>(p.sink + ((int64_t)slot * p.n_sink + pos) * kD);
    dst[lane] = chunk0;
    if (lane < kD / 8 - 64) dst[64 + lane] = chunk1;
  }
  if (pos >= p.slot_len_after[slot] - p.n_recent) {
    uint4* dst = reinterpret_cast<uint4*>(p.recent + ((int64_t)slot * p.n_recent + pos % p.n_recent) * kD);
    dst[lane] = chunk0;
    if (lane < kD / 8 - 64) dst[64 + lane] = chunk1;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  if (p.n_tokens <= 0) return hipSuccess;
  const int blocks = (p.n_tokens + 3) / 4;
  AppendParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(append_kernel), dim3(blocks), dim3(256), args, 0, stream);
}

}  // namespace mla
