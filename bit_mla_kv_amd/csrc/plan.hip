// Split planning and the log-sum-exp combine for the low-bit MLA decode.
//
// plan_kernel (one workgroup) turns the device-resident sequence lengths into
// a balanced work list: every sequence's packed range [n_sink, N - n_recent)
// is cut into page-aligned chunks of one common size P = ceil(total packed
// pages / target items), and every sequence gets one more item for its bf16
// (sink + recent) tokens.  Items are ordered full chunks first, then the
// shorter tail chunks, then the bf16 items, so the hardware's in-order
// dispatch starts the longest work first.  combine_kernel merges each
// sequence's partial results exactly (max-shifted sums), adding the deferred
// zero terms, and writes bf16 outputs and natural-log lse.
#include <algorithm>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

constexpr int kPlanThreads = 64;  // one wave: scans are lane shuffles, no workgroup barriers

__device__ __forceinline__ int seq_packed_pages(const DecodeParams& p, int b, int* first_page) {
  int N = p.seq_len[b];
  const int slot = p.seq_slot[b];
  if (slot < 0 || slot >= p.num_slots) N = 0;
  const int p_lo = p.n_sink, p_hi = N - p.n_recent;
  *first_page = p_lo / kPageTokens;
  return p_hi > p_lo ? (p_hi - 1) / kPageTokens - *first_page + 1 : 0;
}

// exclusive scan over the 64 lanes of the wave; *total gets the sum
__device__ __forceinline__ int wave_exclusive_scan(int v, int* total) {
  const int lane = threadIdx.x;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  *total = __shfl(x, 63, 64);
  return x - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeParams p) {
  const int t = threadIdx.x;
  // total packed pages
  long long local = 0;
  for (int b = t; b < p.batch; b += kPlanThreads) {
    int fp;
    local += seq_packed_pages(p, b, &fp);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) local += __shfl_xor(local, d, 64);
  const long long total = local;
  int pps = (int)std::min<long long>((total + p.target_items - 1) / std::max(1, p.target_items), 1 << 20);
  pps = std::max(pps, p.min_pages_per_split);
  if (p.force_pages_per_split > 0) pps = p.force_pages_per_split;

  // pass 1: counts of full / tail items, scanned in chunks of 64 sequences (lane t owns sequence
  // b0 + t in both passes, so it reads back only what it wrote itself)
  int full_base = 0, tail_base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += kPlanThreads) {
    const int b = b0 + t;
    int nf = 0, nt = 0, fp = 0;
    if (b < p.batch) {
      const int n = seq_packed_pages(p, b, &fp);
      nf = n / pps;
      nt = (n % pps) != 0;
    }
    int tf, tt;
    const int of = wave_exclusive_scan(nf, &tf);
    const int ot = wave_exclusive_scan(nt, &tt);
    if (b < p.batch) {
      p.seq_info[4 * b + 0] = full_base + of;  // first full item
      p.seq_info[4 * b + 1] = nf;
      p.seq_info[4 * b + 2] = nt ? tail_base + ot : -1;
      p.seq_info[4 * b + 3] = fp;              // first packed page (temporarily)
    }
    full_base += tf;
    tail_base += tt;
  }
  const int F = full_base, T = tail_base;
  // pass 2: emit items (b, first page, pages, kind)
  for (int b = t; b < p.batch; b += kPlanThreads) {
    const int fo = p.seq_info[4 * b + 0], nf = p.seq_info[4 * b + 1], tl = p.seq_info[4 * b + 2];
    const int fp = p.seq_info[4 * b + 3];
    int fp2;
    const int n = seq_packed_pages(p, b, &fp2);
    // capacity guards only matter when a caller breaks the seq_len <= max_seq_len contract
    for (int k = 0; k < nf && fo + k < p.max_items; ++k)
      reinterpret_cast<int4*>(p.items)[fo + k] = make_int4(b, fp + k * pps, pps, 0);
    if (tl >= 0) {
      if (F + tl < p.max_items) reinterpret_cast<int4*>(p.items)[F + tl] = make_int4(b, fp + nf * pps, n - nf * pps, 0);
      p.seq_info[4 * b + 2] = F + tl < p.max_items ? F + tl : -1;
    }
    if (F + T + b < p.max_items) reinterpret_cast<int4*>(p.items)[F + T + b] = make_int4(b, 0, 0, 1);
    p.seq_info[4 * b + 3] = F + T + b < p.max_items ? F + T + b : -1;  // bf16 item
    if (fo + nf > p.max_items) p.seq_info[4 * b + 1] = max(0, p.max_items - fo);
  }
  if (t == 0) {
    p.plan_hdr[0] = F + T + p.batch;  // item count
    p.plan_hdr[1] = pps;
  }
}

__device__ __forceinline__ uint16_t f2bf_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// one workgroup per (sequence, head): 128 threads x 4 channels.  A sequence's partial rows are
// merged eight at a time: the loads of a batch are all requested before any is used, and the
// batch joins a running max-shifted sum.
__global__ __launch_bounds__(128) void combine_kernel(DecodeParams p) {
  constexpr int kBatch = 8;
  const int b = blockIdx.x / p.heads;
  const int h = blockIdx.x % p.heads;
  const int t = threadIdx.x;
  const int fo = p.seq_info[4 * b + 0], nf = p.seq_info[4 * b + 1];
  const int tl = p.seq_info[4 * b + 2], bi = p.seq_info[4 * b + 3];
  const int n_rows = nf + (tl >= 0) + (bi >= 0);
  auto item_of = [&](int k) { return k < nf ? fo + k : (k == nf && tl >= 0 ? tl : bi); };
  const int g = t / 16;  // channels 4t..4t+3 lie in group t/16

  float M = -__builtin_inff(), den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n_rows; k0 += kBatch) {
    float mv[kBatch], lv[kBatch];
    f32x4 ov[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = min(k0 + j, n_rows - 1);  // past the end: re-read the last row, weight 0
      const int64_t row = (int64_t)item_of(k) * p.heads + h;
      mv[j] = p.ws_ml[2 * row];
      lv[j] = k0 + j < n_rows ? p.ws_ml[2 * row + 1] : 0.f;
      ov[j] = *reinterpret_cast<const f32x4*>(p.ws_o + row * kDc + 4 * t);
      if (p.has_z) ov[j] += p.ws_z[row * 8 + g];
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (lv[j] > 0.f) mb = fmaxf(mb, mv[j]);
    if (mb == -__builtin_inff()) continue;  // nothing valid yet
    const float r = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - mb);
    acc *= r;
    den *= r;
    M = mb;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (!(lv[j] > 0.f)) continue;
      const float wgt = __builtin_amdgcn_exp2f(mv[j] - M);
      den += wgt * lv[j];
      acc += wgt * ov[j];
    }
  }
  float L = -__builtin_inff();
  if (M != -__builtin_inff()) {
    acc *= 1.f / den;
    L = M + __log2f(den);
  }
  uint16_t* o = p.out + ((int64_t)b * p.heads + h) * kDc + 4 * t;
  uint2 packed;
  packed.x = (uint32_t)f2bf_rne(acc[0]) | ((uint32_t)f2bf_rne(acc[1]) << 16);
  packed.y = (uint32_t)f2bf_rne(acc[2]) | ((uint32_t)f2bf_rne(acc[3]) << 16);
  *reinterpret_cast<uint2*>(o) = packed;
  if (p.lse && t == 0) p.lse[(int64_t)b * p.heads + h] = L * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_plan(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.batch * p.heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
