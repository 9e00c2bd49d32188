// Split-KV low-bit MLA decode for gfx950 (CDNA4): work decomposition and kernel choice.
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
// Some splits hold page-aligned chunks of the packed range, the others chunks
// of the bf16 token list (plan_kernel sizes both from the device-resident
// lengths).
// Each split leaves an unnormalised partial output with its running max and
// sum, and the zero-term sums; combine_kernel merges them exactly.
//
// Head groups: 64 heads per workgroup (decode64.hip) when the head count is a
// multiple of 64, else 16 (decode16.hip): with 64 heads sharing a latent the
// decode is MFMA-bound and the unpacked codes are shared by wave roles; with
// 16 it is HBM-bound and every wave streams its own rows of the pages.
#include <algorithm>
#include <cstdlib>

#include "decode_common.h"

namespace mla {

bool decode_config(int heads, int n_sink, int n_recent, int batch, int max_seq_len, DecodeConfig* cfg) {
  if (heads > 0 && heads % 64 != 0 && heads % 16 == 0) {
    cfg->heads_per_wg = 16; cfg->threads = 256; cfg->wg_per_cu = 1;
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
  // per sequence: packed pages, and bf16 tokens in 64-token pages (at least one bf16 item each)
  const int64_t max_pp = std::max<int64_t>(0, ((int64_t)max_seq_len - n_recent + kPageTokens - 1) / kPageTokens);
  const int64_t max_bp = ((int64_t)bf16_token_count(max_seq_len, n_sink, n_recent) + kPageTokens - 1) / kPageTokens;
  const int64_t min_chunk = cfg->force_pages_per_split > 0 ? cfg->force_pages_per_split : cfg->min_pages_per_split;
  int64_t items = (int64_t)batch * ((max_pp + min_chunk - 1) / min_chunk + std::max<int64_t>(1, (max_bp + min_chunk - 1) / min_chunk));
  // full chunks (packed and bf16) <= total pages / chunk <= target, plus at most one packed tail
  // and one short or empty bf16 item per sequence
  if (cfg->force_pages_per_split <= 0) items = std::min<int64_t>(items, cfg->target_items + 2 * (int64_t)batch);
  cfg->max_items = (int)std::min<int64_t>(items, 1 << 30);
  return true;
}

hipError_t prepare_decode(const DecodeParams& p, int bits_c) {
  const int hpw = p.heads / p.head_groups;
  const int64_t blocks = ((int64_t)p.max_items + 7) / 8 * 8 * p.head_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (hpw == 64) return prepare_decode64(p, bits_c);
  if (hpw == 16) return (bits_c == 4 || bits_c == 2) ? hipSuccess : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int bits_c, hipStream_t stream) {
  const int hpw = p.heads / p.head_groups;
  if (hpw == 64) return launch_decode64(p, bits_c, stream);
  if (hpw == 16) return launch_decode16(p, bits_c, stream);
  return hipErrorInvalidValue;
}

}  // namespace mla
