// Device helpers shared by the decode kernels (gfx950).
#pragma once
#include "mla_internal.h"

namespace mla {
namespace dev {

typedef _Float16 f16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

__device__ __forceinline__ float bf16f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// position offset p (0..7) inside an 8-channel block -> channel offset, as the
// unpacking below orders them (content codes of the layout's width; RoPE codes are 4 bit)
template <int BITS>
__device__ __forceinline__ constexpr int perm8(int p) {
  return BITS == 4 ? ((p & 3) * 2 + (p >> 2)) : ((p & 1) * 4 + (p >> 1));
}

// 8 nibbles (channels 0..7 of a dword) -> exact fp16 codes in perm8<4> order
__device__ __forceinline__ uint4 unpack4(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// 16 crumbs (channels 0..15 of a dword) -> two groups of 8 exact fp16 codes in perm8<2> order
__device__ __forceinline__ void unpack2(uint32_t w, uint4& first, uint4& second) {
  const uint32_t b0 = w & 0x03030303u, b1 = (w >> 2) & 0x03030303u;
  const uint32_t b2 = (w >> 4) & 0x03030303u, b3 = (w >> 6) & 0x03030303u;
  first = make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, 512.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, 512.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b2, 512.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b3, 512.0f, false)));
  second = make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b0, 512.0f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b1, 512.0f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b2, 512.0f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b3, 512.0f, true)));
}

// 8 bf16 values (one 16-byte chunk, channels 0..7) -> fp16 in the order perm8<BITS>
template <int BITS>
__device__ __forceinline__ uint4 bf16_chunk_to_f16(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  f16 h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = perm8<BITS>(j);
    const uint32_t bits = (c & 1) ? (w[c >> 1] >> 16) : (w[c >> 1] & 0xFFFFu);
    h[j] = (f16)bf16f(bits);
  }
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, f16x2{h[0], h[1]});
  r.y = __builtin_bit_cast(uint32_t, f16x2{h[2], h[3]});
  r.z = __builtin_bit_cast(uint32_t, f16x2{h[4], h[5]});
  r.w = __builtin_bit_cast(uint32_t, f16x2{h[6], h[7]});
  return r;
}

__device__ __forceinline__ f16x8 lds_read8(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }

// Explicit LDS (address space 3) pointers.  An LDS address can be passed through an empty asm
// statement (to keep address arithmetic from being hoisted out of a loop) without losing its
// address space, which a generic pointer would (turning ds_read into flat loads).
template <typename T>
using lds_ptr = __attribute__((address_space(3))) T*;

template <typename T>
__device__ __forceinline__ lds_ptr<T> lds_opaque(T* generic) {
  uint32_t off = (uint32_t)reinterpret_cast<uintptr_t>(generic);  // low bits of a generic LDS address
  asm volatile("" : "+v"(off));
  return reinterpret_cast<lds_ptr<T>>(static_cast<uintptr_t>(off));
}

template <typename T, typename P>
__device__ __forceinline__ T lds_load(lds_ptr<P> p) {
  return *reinterpret_cast<lds_ptr<const T>>(p);
}

__device__ __forceinline__ f16x4 lds_tr4(const f16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(f16x4, v);
}

__device__ __forceinline__ f16x4 lds_tr4(lds_ptr<f16> p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_ptr<i16x4>>(p));
  return __builtin_bit_cast(f16x4, v);
}

__device__ __forceinline__ f16x8 cat8(f16x4 lo, f16x4 hi) {
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fmax4(f32x4 v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }


// Handshake flags between the waves of a workgroup live in LDS, read and written as volatile words.
typedef __attribute__((address_space(3))) volatile int lds_vint;
// Returns 1 when the wait gave up after `spin` polls (counted into the workspace header).
// The empty asm with a memory clobber keeps the compiler from moving the LDS reads of the data the
// flag guards above the wait.
__device__ __forceinline__ int wait_at_least(lds_vint* flag, int target, int spin) {
  int gave_up = 1;
  for (int i = 0; i < spin; ++i) {
    if (__builtin_amdgcn_readfirstlane(*flag) >= target) {
      gave_up = 0;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  return gave_up;
}
// publish a flag value once this wave's earlier LDS writes have completed
__device__ __forceinline__ void signal(lds_vint* flag, int value, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) *flag = value;
}

// ---- split-plan facts about sequence b, shared by the planner, the decode kernels and the combine
__device__ __forceinline__ int seq_packed_pages(const DecodeParams& p, int b, int* first_page) {
  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  const int p_lo = p.n_sink, p_hi = N - p.n_recent;
  *first_page = p_lo / kPageTokens;
  return p_hi > p_lo ? (p_hi - 1) / kPageTokens - *first_page + 1 : 0;
}
// the sequence's bf16 tokens (sink, then the recent window) and their count in 64-token pages
__device__ __forceinline__ int seq_bf16_tokens(const DecodeParams& p, int b) {
  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  return bf16_token_count(N, p.n_sink, p.n_recent);
}
__device__ __forceinline__ int seq_bf16_pages(const DecodeParams& p, int b) {
  return (seq_bf16_tokens(p, b) + kPageTokens - 1) / kPageTokens;
}
// bf16 items of a sequence with chunks of pps pages: at least one (an empty sequence still leaves
// a partial row for the combine)
__device__ __forceinline__ int bf16_items(int bf_pages, int pps) { return max(1, (bf_pages + pps - 1) / pps); }

// Sequence b is decoded by one work item (no packed chunk, one bf16 chunk, and that item is in the
// list): that item's workgroups write the final outputs and lse themselves and the combine leaves
// the sequence alone.  Read after the plan kernel has run.
__device__ __forceinline__ bool decoded_in_one_item(const DecodeParams& p, int b) {
  int fp;
  return p.seq_info[4 * b + 3] >= 0 && seq_packed_pages(p, b, &fp) == 0 &&
         bf16_items(seq_bf16_pages(p, b), p.plan_hdr[kHdrPagesPerSplit]) == 1;
}

__device__ __forceinline__ uint16_t f2bf_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// four outputs as bf16 (round to nearest even), one 8-byte store
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, f32x4 v) {
  uint2 q;
  q.x = (uint32_t)f2bf_rne(v[0]) | ((uint32_t)f2bf_rne(v[1]) << 16);
  q.y = (uint32_t)f2bf_rne(v[2]) | ((uint32_t)f2bf_rne(v[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = q;
}

}  // namespace dev
}  // namespace mla
