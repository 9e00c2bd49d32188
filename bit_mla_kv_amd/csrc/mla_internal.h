// Internal declarations shared by the host ABI and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kDc = 512;         // content latent width
constexpr int kDr = 64;          // RoPE key width
constexpr int kD = kDc + kDr;    // row width
constexpr int kGroup = 64;       // quantization group
constexpr int kGroups = kD / kGroup;  // 9: eight content groups, one RoPE-key group
constexpr int kPageTokens = 64;  // tokens per page

__host__ __device__ inline int content_row_bytes(int bits_c) { return kDc * bits_c / 8; }
__host__ __device__ inline int page_bytes(int bits_c) {
  return kPageTokens * (content_row_bytes(bits_c) + kDr / 2 + 4 * kGroups);
}

// Number of a sequence's tokens read from bf16: the first min(n_sink, N), then the recent window
// [max(n_sink, N - n_recent), N); each token once.
__host__ __device__ inline int bf16_token_count(int N, int n_sink, int n_recent) {
  const int ns = N < n_sink ? N : n_sink;
  const int rstart = n_sink > N - n_recent ? n_sink : N - n_recent;
  return ns + (N - rstart > 0 ? N - rstart : 0);
}

// Words of the decode workspace header (int32).  plan_kernel writes them at the start of every
// decode call; the decode kernels add to the counters.
constexpr int kHdrItems = 0;          // work items of this call
constexpr int kHdrPagesPerSplit = 1;  // pages per packed chunk
constexpr int kHdrDirect = 2;        // workgroups that wrote their sequence's final output (one-item sequences)
constexpr int kHdrGiveUps = 4;        // handshake waits between two waves that gave up (bounded wait)
constexpr int kHdrBadPages = 5;       // page reads whose block-table entry lay outside the table or pool
constexpr int kHdrBadSeqs = 6;        // sequences with a slot outside the cache or a length outside [0, max_seq_len]
constexpr int kHdrDropped = 7;        // work items dropped for lack of workspace rows
constexpr int kDefaultSpin = 1 << 18; // polls of a bounded handshake wait

struct AppendParams {
  uint8_t* pages;
  int64_t num_pages;
  uint16_t* sink;
  uint16_t* recent;
  int32_t num_slots;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t n_sink, n_recent;
  int32_t bits_c;
  const uint16_t* kv;
  const int32_t* token_slot;
  const int32_t* token_pos;
  const int32_t* slot_len_after;
  int32_t n_tokens;
};

struct DecodeParams {
  const uint8_t* pages;
  int64_t num_pages;
  const uint16_t* sink;
  const uint16_t* recent;
  int32_t num_slots;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t n_sink, n_recent;
  const uint16_t* q;          // [batch][H][576]
  const int32_t* seq_slot;
  const int32_t* seq_len;
  int32_t batch, heads;       // heads: rows per sequence = q_len * heads_per_query
  int32_t max_seq_len;        // the caller's bound on seq_len (sizes the workspace)
  int32_t spin_limit;         // polls before a handshake wait gives up (counted in the header)
  int32_t q_len;              // query tokens per sequence; row r is query r / heads_per_query
  int32_t heads_per_query;    // a multiple of 16, so a 16-row block belongs to one query
  float scale_log2e;          // softmax_scale * log2(e)
  int32_t head_groups;        // heads / heads-per-workgroup
  // split plan (written on the device by plan_kernel)
  int32_t target_items;       // aimed-at number of packed work items (about one per resident workgroup)
  int32_t min_pages_per_split;
  int32_t force_pages_per_split;  // > 0: fixed chunk size (tests / tuning)
  int32_t max_items;          // capacity of items / partial rows
  int32_t* items;             // [max_items] int4 (sequence, first page, pages, kind 0 packed / 1 bf16)
  int32_t* seq_info;          // [batch] int4 (first full item, full items, tail item or -1, bf16 item)
  int32_t* plan_hdr;          // header words kHdr* (item count, pages per chunk, counters)
  float* ws_o;                // [max_items][H][512]: unnormalised partial outputs sum_t 2^(x_t - m) v_t
  float* ws_ml;               // [max_items][H][2]: running max m (log2 domain) and sum l (l = 0: empty)
  float* ws_z;                // [max_items][H][8]: zero-term sums sum_t 2^(x_t - m) z_t,g (has_z)
  int32_t has_z;              // ws_z holds zero terms still to be added to each group's channels
  uint16_t* out;              // [batch][H][512] bf16
  float* lse;                 // [batch][H] natural log, may be null
};

// Kernel launchers (each returns the hipError_t of its launch).  prepare_decode* set the kernel
// attributes a decode launch needs and check its grid; they enqueue nothing, so the host entry
// points call them before the first launch of a call.
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t prepare_decode(const DecodeParams& p, int bits_c);
hipError_t prepare_decode64(const DecodeParams& p, int bits_c);
hipError_t launch_decode(const DecodeParams& p, int bits_c, hipStream_t stream);
hipError_t launch_decode64(const DecodeParams& p, int bits_c, hipStream_t stream);
hipError_t launch_decode16(const DecodeParams& p, int bits_c, hipStream_t stream);
hipError_t launch_plan(const DecodeParams& p, hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);

// Decode configuration shared by the workspace query and the launch.
struct DecodeConfig {
  int heads_per_wg;      // heads covered by one workgroup
  int threads;           // workgroup size
  int wg_per_cu;         // expected resident workgroups per CU
  int target_items;      // packed work items the plan aims at
  int min_pages_per_split;
  int force_pages_per_split;
  int max_items;         // bound on plan items (workspace rows, grid)
};
bool decode_config(int heads, int n_sink, int n_recent, int batch, int max_seq_len, DecodeConfig* cfg);

}  // namespace mla
