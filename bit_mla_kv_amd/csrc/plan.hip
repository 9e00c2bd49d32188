// Split planning and the log-sum-exp combine for the low-bit MLA decode.
//
// plan_kernel (one workgroup) turns the device-resident sequence lengths into
// a balanced work list: every sequence's packed range [n_sink, N - n_recent)
// is cut into page-aligned chunks of one common size P = ceil(total pages /
// target items), and its list of bf16 (sink + recent) tokens into chunks of
// 64 P tokens (one item when, as usual, there are at most 132; many when the
// recent window is long).  Items are ordered bf16 chunks first (short: their
// CUs go on to packed work), then the full chunks, then the tail chunks
// longest first, so the hardware's in-order dispatch is a greedy
// longest-first schedule of the packed work.  When a slightly longer chunk lets
// every packed item run at once (one round of workgroups), that chunk is used.  combine_kernel merges each
// sequence's partial results exactly (max-shifted sums), adding the deferred
// zero terms, and writes bf16 outputs and natural-log lse; a sequence decoded in
// one work item has had its outputs written by the decode kernel and is skipped.
#include <algorithm>

#include "decode_common.h"

namespace mla {
namespace {
using namespace dev;

constexpr int kPlanThreads = 64;  // one wave: scans are DPP row operations, no workgroup barriers
constexpr int kPlanRegs = 8;      // sequence lengths a lane keeps in registers for the chunk search

// Cross-lane scans and sums of the plan wave with DPP row operations (plain VALU instructions; a
// ds_bpermute shuffle costs an LDS round trip, and the plan is a chain of such steps).  Inclusive
// scan in lane order: shifts by 1, 2, 4, 8 within each 16-lane row, then the last lane of rows 0
// and 2 into rows 1 and 3 (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31).  Lanes a
// shift leaves without a source, and rows outside the row mask, take the identity (old value).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_in(int x, int identity) {
  return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ long long dpp_in(long long x, long long identity) {
  const int lo = __builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(identity >> 32), (int)(x >> 32), CTRL, ROW_MASK, 0xf, false);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_inclusive(T x, T identity, Op op) {
  x = op(x, dpp_in<0x111, 0xf>(x, identity));  // row_shr:1
  x = op(x, dpp_in<0x112, 0xf>(x, identity));  // row_shr:2
  x = op(x, dpp_in<0x114, 0xf>(x, identity));  // row_shr:4
  x = op(x, dpp_in<0x118, 0xf>(x, identity));  // row_shr:8
  x = op(x, dpp_in<0x142, 0xa>(x, identity));  // row_bcast:15 into rows 1, 3
  x = op(x, dpp_in<0x143, 0xc>(x, identity));  // row_bcast:31 into rows 2, 3
  return x;
}
__device__ __forceinline__ int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }
__device__ __forceinline__ long long lane63(long long x) {
  const int lo = __builtin_amdgcn_readlane((int)x, 63), hi = __builtin_amdgcn_readlane((int)(x >> 32), 63);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return lane63(wave_inclusive(v, T(0), [](T a, T b) { return a + b; }));
}
__device__ __forceinline__ int wave_max(int v, int identity) {
  return lane63(wave_inclusive(v, identity, [](int a, int b) { return max(a, b); }));
}
// exclusive scan over the 64 lanes of the wave; *total gets the sum
__device__ __forceinline__ int wave_exclusive_scan(int v, int* total) {
  const int x = wave_inclusive(v, 0, [](int a, int b) { return a + b; });
  *total = lane63(x);
  return x - v;
}

// Sequences whose slot lies outside the cache or whose length lies outside [0, max_seq_len] (they
// decode as empty, or may not fit the workspace): counted by the plan from the lengths it reads.
__device__ int count_bad_seqs(const DecodeParams& p, int t) {
  int bad = 0;
  for (int b = t; b < p.batch; b += kPlanThreads) {
    const int N = p.seq_len[b], slot = p.seq_slot[b];
    bad += (slot < 0 || slot >= p.num_slots || N < 0 || N > p.max_seq_len) ? 1 : 0;
  }
  return wave_sum(bad);
}

// The header counters: the decode kernels add to the first three.
__device__ void write_counters(const DecodeParams& p, int t, int bad) {
  if (t == 0) {
    p.plan_hdr[kHdrGiveUps] = 0;  // the decode kernels add to these three
    p.plan_hdr[kHdrBadPages] = 0;
    p.plan_hdr[kHdrDirect] = 0;
    p.plan_hdr[kHdrBadSeqs] = bad;
  }
}

// The plan for batch <= kPlanThreads * kPlanRegs: every sequence's length is read once into lane
// registers (sequence t + 64 k in register k), and both passes run on them.
__device__ void plan_in_registers(const DecodeParams& p, int t) {
  constexpr int R = kPlanRegs;
  int fpg[R], npk[R], nbt[R];
  bool has[R];
  int Nv[R], sv[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {  // all loads first: one round trip
    const int b = t + kPlanThreads * k;
    has[k] = b < p.batch;
    Nv[k] = has[k] ? p.seq_len[b] : 0;
    sv[k] = has[k] ? p.seq_slot[b] : 0;
  }
  long long local = 0;
  int n_max = 0, bad = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    bad += has[k] && (sv[k] < 0 || sv[k] >= p.num_slots || Nv[k] < 0 || Nv[k] > p.max_seq_len);
    const int N = (sv[k] < 0 || sv[k] >= p.num_slots) ? 0 : Nv[k];
    const int p_lo = p.n_sink, p_hi = N - p.n_recent;
    fpg[k] = p_lo / kPageTokens;
    npk[k] = has[k] && p_hi > p_lo ? (p_hi - 1) / kPageTokens - fpg[k] + 1 : 0;
    nbt[k] = has[k] ? bf16_token_count(N, p.n_sink, p.n_recent) : 0;
    local += npk[k] + (nbt[k] + kPageTokens - 1) / kPageTokens;
    n_max = std::max(n_max, npk[k]);
  }
  local = wave_sum(local);
  n_max = wave_max(n_max, 0);
  write_counters(p, t, wave_sum(bad));
  int pps = (int)std::min<long long>((local + p.target_items - 1) / std::max(1, p.target_items), 1 << 20);
  pps = std::max(pps, p.min_pages_per_split);
  // target_items workgroups run at once.  Full chunks plus tails can exceed it by up to batch, and
  // the excess then runs as a second round after a full chunk.  When a chunk at most a quarter
  // longer brings every packed item into one round, take the shortest such chunk (the bf16 items
  // are short and run first, so their CUs go on to packed chunks: they take no slot of the round).
  if (2 * p.batch <= p.target_items) {
    auto items_at = [&](int c) {
      int n = 0;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (kPlanThreads * k >= p.batch) break;  // (integer divisions are not cheap)
        n += (npk[k] + c - 1) / c;
      }
      return wave_sum(n);
    };
    int lo = pps, hi = std::min(std::max(n_max, pps), pps + pps / 4);
    if (items_at(lo) > p.target_items && items_at(hi) <= p.target_items) {
      while (hi - lo > 1) {  // items_at(lo) > target_items >= items_at(hi); items_at is non-increasing
        const int mid = lo + (hi - lo) / 2;
        if (items_at(mid) <= p.target_items) hi = mid;
        else lo = mid;
      }
      pps = hi;
    }
  }
  if (p.force_pages_per_split > 0) pps = p.force_pages_per_split;

  // pass 1: per-sequence item counts and their offsets (scans over each group of 64 sequences)
  int fo[R], nf[R], tl[R], tp[R], nbi[R], bo[R];
  int full_base = 0, tail_base = 0, bf_base = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (kPlanThreads * k >= p.batch) {
      nf[k] = tp[k] = nbi[k] = fo[k] = tl[k] = bo[k] = 0;
      continue;
    }
    nf[k] = npk[k] / pps;
    tp[k] = npk[k] - nf[k] * pps;  // tail pages (0: no tail)
    nbi[k] = has[k] ? bf16_items((nbt[k] + kPageTokens - 1) / kPageTokens, pps) : 0;
    int tf, tt, tb;
    const int of = wave_exclusive_scan(nf[k], &tf);
    const int ot = wave_exclusive_scan(tp[k] != 0, &tt);
    const int ob = wave_exclusive_scan(nbi[k], &tb);
    fo[k] = full_base + of;
    tl[k] = tail_base + ot;  // sequence order, replaced by the longest-first rank below
    bo[k] = bf_base + ob;
    full_base += tf;
    tail_base += tt;
    bf_base += tb;
  }
  const int F = full_base, T = tail_base, BF = bf_base;
  // Tail chunks longest first: the hardware starts workgroups in item order as CUs free up, so
  // this is greedy longest-processing-time scheduling of the tails after the equal full chunks.
  // A tail's position is its rank by (pages descending, sequence ascending), for up to
  // kTailSortMax sequences (otherwise the tails keep sequence order).
  constexpr int kTailSortMax = 4 * kPlanThreads;
  if (p.batch <= kTailSortMax) {
    const int n_groups = (p.batch + kPlanThreads - 1) / kPlanThreads;
    int ranks[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      if (k2 >= n_groups) break;
      const int n_src = min(kPlanThreads, p.batch - kPlanThreads * k2);
      for (int src = 0; src < n_src; ++src) {
        const int other = __builtin_amdgcn_readlane(tp[k2], src), b2 = src + kPlanThreads * k2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k >= n_groups) break;
          const int mine = tp[k], b = t + kPlanThreads * k;
          ranks[k] += other > mine || (other == mine && other > 0 && b2 < b);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) tl[k] = ranks[k];
  }
  // pass 2: emit items (b, first page, pages, kind): bf16 chunks, full chunks, tails
  const int chunk = pps * kPageTokens;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (!has[k]) continue;
    const int b = t + kPlanThreads * k;
    // capacity guards only matter when a caller breaks the seq_len <= max_seq_len contract
    for (int j = 0; j < nf[k] && BF + fo[k] + j < p.max_items; ++j)
      reinterpret_cast<int4*>(p.items)[BF + fo[k] + j] = make_int4(b, fpg[k] + j * pps, pps, 0);
    int ti = -1;
    if (tp[k] != 0) {
      ti = BF + F + tl[k];
      if (ti < p.max_items) reinterpret_cast<int4*>(p.items)[ti] = make_int4(b, fpg[k] + nf[k] * pps, tp[k], 0);
      else ti = -1;
    }
    for (int j = 0; j < nbi[k] && bo[k] + j < p.max_items; ++j)
      reinterpret_cast<int4*>(p.items)[bo[k] + j] = make_int4(b, j * chunk, min(chunk, nbt[k] - j * chunk), 1);
    const int nf_cap = BF + fo[k] + nf[k] > p.max_items ? max(0, p.max_items - BF - fo[k]) : nf[k];
    reinterpret_cast<int4*>(p.seq_info)[b] = make_int4(BF + fo[k], nf_cap, ti, bo[k] < p.max_items ? bo[k] : -1);
  }
  if (t == 0) {
    p.plan_hdr[kHdrItems] = F + T + BF;
    p.plan_hdr[kHdrPagesPerSplit] = pps;
    p.plan_hdr[kHdrDropped] = max(0, F + T + BF - p.max_items);
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeParams p) {
  const int t = threadIdx.x;
  if (p.batch <= kPlanThreads * kPlanRegs) {
    plan_in_registers(p, t);
    return;
  }
  // larger batches: the sequences are read per pass, chunks of P = ceil(total pages / target
  // items) pages, tails in sequence order
  write_counters(p, t, count_bad_seqs(p, t));
  long long local = 0;
  for (int b = t; b < p.batch; b += kPlanThreads) {
    int fp;
    local += seq_packed_pages(p, b, &fp) + seq_bf16_pages(p, b);
  }
  local = wave_sum(local);
  int pps = (int)std::min<long long>((local + p.target_items - 1) / std::max(1, p.target_items), 1 << 20);
  pps = std::max(pps, p.min_pages_per_split);
  if (p.force_pages_per_split > 0) pps = p.force_pages_per_split;

  // pass 1: counts of full / tail / bf16 items, scanned in chunks of 64 sequences (lane t owns
  // sequence b0 + t in both passes, so it reads back only what it wrote itself)
  int full_base = 0, tail_base = 0, bf_base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += kPlanThreads) {
    const int b = b0 + t;
    int nf = 0, nt = 0, nbi = 0, fp = 0;
    if (b < p.batch) {
      const int n = seq_packed_pages(p, b, &fp);
      nf = n / pps;
      nt = (n % pps) != 0;
      nbi = bf16_items(seq_bf16_pages(p, b), pps);
    }
    int tf, tt, tb;
    const int of = wave_exclusive_scan(nf, &tf);
    const int ot = wave_exclusive_scan(nt, &tt);
    const int ob = wave_exclusive_scan(nbi, &tb);
    if (b < p.batch) {
      p.seq_info[4 * b + 0] = full_base + of;  // first full item
      p.seq_info[4 * b + 1] = nf;
      p.seq_info[4 * b + 2] = nt ? tail_base + ot : -1;
      p.seq_info[4 * b + 3] = bf_base + ob;    // first bf16 item, relative (temporarily)
    }
    full_base += tf;
    tail_base += tt;
    bf_base += tb;
  }
  const int F = full_base, T = tail_base, BF = bf_base;
  // pass 2: emit items (b, first page, pages, kind)
  for (int b = t; b < p.batch; b += kPlanThreads) {
    const int fo = p.seq_info[4 * b + 0], nf = p.seq_info[4 * b + 1];
    const int tl = p.seq_info[4 * b + 2];
    const int bo = p.seq_info[4 * b + 3];
    int fp;
    const int n = seq_packed_pages(p, b, &fp);
    // capacity guards only matter when a caller breaks the seq_len <= max_seq_len contract
    for (int k = 0; k < nf && BF + fo + k < p.max_items; ++k)
      reinterpret_cast<int4*>(p.items)[BF + fo + k] = make_int4(b, fp + k * pps, pps, 0);
    if (tl >= 0) {
      const int ti = BF + F + tl;
      if (ti < p.max_items) reinterpret_cast<int4*>(p.items)[ti] = make_int4(b, fp + nf * pps, n - nf * pps, 0);
      p.seq_info[4 * b + 2] = ti < p.max_items ? ti : -1;
    }
    // bf16 chunks (first index into the sequence's bf16 token list, count)
    const int nbt = seq_bf16_tokens(p, b), chunk = pps * kPageTokens;
    const int nbi = bf16_items(seq_bf16_pages(p, b), pps);
    for (int k = 0; k < nbi && bo + k < p.max_items; ++k)
      reinterpret_cast<int4*>(p.items)[bo + k] = make_int4(b, k * chunk, min(chunk, nbt - k * chunk), 1);
    p.seq_info[4 * b + 3] = bo < p.max_items ? bo : -1;  // first bf16 item
    p.seq_info[4 * b + 0] = BF + fo;
    if (BF + fo + nf > p.max_items) p.seq_info[4 * b + 1] = max(0, p.max_items - BF - fo);
  }
  if (t == 0) {
    p.plan_hdr[kHdrItems] = F + T + BF;
    p.plan_hdr[kHdrPagesPerSplit] = pps;
    p.plan_hdr[kHdrDropped] = max(0, F + T + BF - p.max_items);
  }
}

// One workgroup of 4 waves per (sequence, head).  Wave w merges the sequence's partial rows
// w, w + 4, ... over all 512 channels (8 per lane), eight rows at a time with every load
// requested before use, as a running max-shifted sum; the four waves' sums are then joined
// through LDS.
// rw waves per output row (sequence b, head h), W / rw rows per workgroup of W waves: wave w takes
// row blockIdx.x * (W / rw) + w / rw and, of that row's partials (one per work item of the sequence),
// those with index = w % rw modulo rw, four at a time, merged with a running max; the waves of a
// row are joined through LDS.  Lane l holds channels 4 l .. 4 l + 3 (group l / 16) and
// 256 + 4 l .. (group 4 + l / 16).  rw (1 .. 16, a power of two) is chosen on the host so that a
// launch has a few thousand waves in flight and a wave merges about one batch of partials: one
// wave per row when the rows are many, up to sixteen when they are few (and their partials many).
template <int W>
__global__ __launch_bounds__(64 * W) void combine_kernel(DecodeParams p, int rw) {
  constexpr int kBatch = 4;  // partials requested together: 4 keeps the kernel at 74 VGPRs, 6-7 waves
                              // per SIMD, which beat 8 (114 VGPRs, 4 waves) on every shape measured
  __shared__ float sh_m[W], sh_d[W];
  __shared__ f32x4 sh_acc[W][2][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = w % rw, w0 = w - sub;  // w0: the row's first wave
  const int64_t rid = (int64_t)blockIdx.x * (W / rw) + w / rw;
  const bool live = rid < (int64_t)p.batch * p.heads;
  const int b = live ? (int)(rid / p.heads) : 0;
  const int h = live ? (int)(rid % p.heads) : 0;
  const int fo = p.seq_info[4 * b + 0], nf = p.seq_info[4 * b + 1];
  const int tl = p.seq_info[4 * b + 2], bi = p.seq_info[4 * b + 3];
  // the sequence's bf16 chunks are consecutive items from bi on (chunks of 64 P tokens)
  const int nbi = bi < 0 ? 0 : min(bf16_items(seq_bf16_pages(p, b), p.plan_hdr[kHdrPagesPerSplit]),
                                   min(p.plan_hdr[kHdrItems], p.max_items) - bi);
  // a sequence decoded in one item has its outputs written by the decode kernel already
  const bool direct = live && decoded_in_one_item(p, b);
  const int n_rows = live && !direct ? nf + (tl >= 0) + nbi : 0;
  auto item_of = [&](int k) {
    return k < nf ? fo + k : (k == nf && tl >= 0 ? tl : bi + (k - nf - (tl >= 0)));
  };
  const int g0 = lane / 16, g1 = 4 + lane / 16;

  float M = -__builtin_inff(), den = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int my_rows = n_rows > sub ? (n_rows - sub + rw - 1) / rw : 0;
  for (int j0 = 0; j0 < my_rows; j0 += kBatch) {
    float mv[kBatch], lv[kBatch];
    f32x4 ov0[kBatch], ov1[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = sub + rw * min(j0 + j, my_rows - 1);  // past the end: the last row again, weight 0
      const int64_t row = (int64_t)item_of(k) * p.heads + h;
      mv[j] = p.ws_ml[2 * row];
      lv[j] = j0 + j < my_rows ? p.ws_ml[2 * row + 1] : 0.f;
      ov0[j] = *reinterpret_cast<const f32x4*>(p.ws_o + row * kDc + 4 * lane);
      ov1[j] = *reinterpret_cast<const f32x4*>(p.ws_o + row * kDc + 256 + 4 * lane);
      if (p.has_z) {
        ov0[j] += p.ws_z[row * 8 + g0];
        ov1[j] += p.ws_z[row * 8 + g1];
      }
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (lv[j] > 0.f) mb = fmaxf(mb, mv[j]);
    if (mb == -__builtin_inff()) continue;  // nothing valid yet
    const float r = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - mb);
    acc0 *= r;
    acc1 *= r;
    den *= r;
    M = mb;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (!(lv[j] > 0.f)) continue;
      const float wgt = __builtin_amdgcn_exp2f(mv[j] - M);
      den += wgt * lv[j];
      acc0 += wgt * ov0[j];
      acc1 += wgt * ov1[j];
    }
  }
  if (rw > 1) {  // join the row's waves in its first wave
    if (lane == 0) {
      sh_m[w] = M;
      sh_d[w] = den;
    }
    sh_acc[w][0][lane] = acc0;
    sh_acc[w][1][lane] = acc1;
    __syncthreads();
    if (sub != 0) return;
    float Mt = M;
    for (int v = 1; v < rw; ++v) Mt = fmaxf(Mt, sh_m[w0 + v]);
    if (Mt != -__builtin_inff()) {
      float dt = 0.f;
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
      for (int v = 0; v < rw; ++v) {
        const float mv = sh_m[w0 + v];
        if (mv == -__builtin_inff()) continue;
        const float f = __builtin_amdgcn_exp2f(mv - Mt);
        dt += f * sh_d[w0 + v];
        o0 += f * sh_acc[w0 + v][0][lane];
        o1 += f * sh_acc[w0 + v][1][lane];
      }
      M = Mt;
      den = dt;
      acc0 = o0;
      acc1 = o1;
    }
  }
  if (!live || direct) return;
  float L = -__builtin_inff();
  if (M != -__builtin_inff()) {
    const float inv = 1.f / den;
    acc0 *= inv;
    acc1 *= inv;
    L = M + __log2f(den);
  }
  uint16_t* o = p.out + rid * kDc;
  store_bf16x4(o + 4 * lane, acc0);
  store_bf16x4(o + 256 + 4 * lane, acc1);
  if (p.lse && lane == 0) p.lse[rid] = L * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_plan(const DecodeParams& p, hipStream_t stream) {
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(plan_kernel), dim3(1), dim3(kPlanThreads), args, 0, stream);
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.heads;
  if (rows == 0) return hipSuccess;
  // waves per row: at least 2,048 waves in all, and (as far as 16 waves go) at most 8 partials per
  // wave, taking max_items / batch for a row's partial count
  const int64_t per_row = ((int64_t)p.max_items + p.batch - 1) / p.batch;
  int rw = 1;
  while (rw < 16 && (rows * rw < 2048 || 8 * rw < per_row)) rw *= 2;
  DecodeParams arg = p;
  int rw_arg = rw;
  void* args[] = {&arg, &rw_arg};
  if (rw <= 4) {
    const int64_t blocks = (rows * rw + 3) / 4;
    return hipLaunchKernel(reinterpret_cast<const void*>(combine_kernel<4>), dim3((unsigned)blocks), dim3(64 * 4),
                           args, 0, stream);
  }
  const int64_t blocks = (rows * rw + 15) / 16;
  return hipLaunchKernel(reinterpret_cast<const void*>(combine_kernel<16>), dim3((unsigned)blocks), dim3(64 * 16),
                         args, 0, stream);
}

}  // namespace mla
