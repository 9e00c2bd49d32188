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
  int32_t batch, heads;
  float scale_log2e;          // softmax_scale * log2(e)
  int32_t pages_per_split;
  int32_t n_splits;           // per sequence: 1 bf16 split + packed splits
  int32_t head_groups;        // heads / heads-per-workgroup
  float* ws_o;                // [batch][n_splits][H][512]: unnormalised partial outputs sum_t 2^(x_t - m) v_t
  float* ws_ml;               // [batch][n_splits][H][2]: running max m (log2 domain) and sum l (l = 0: empty)
  float* ws_z;                // [batch][n_splits][H][8]: zero-term sums sum_t 2^(x_t - m) z_t,g (has_z)
  int32_t has_z;              // ws_z holds zero terms still to be added to each group's channels
  uint16_t* out;              // [batch][H][512] bf16
  float* lse;                 // [batch][H] natural log, may be null
};

// Kernel launchers (each returns the hipError_t of its launch).
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int bits_c, hipStream_t stream);
hipError_t launch_decode128(const DecodeParams& p, int bits_c, hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);

// Decode configuration shared by the workspace query and the launch.
struct DecodeConfig {
  int heads_per_wg;      // heads covered by one workgroup
  int threads;           // workgroup size
  int wg_per_cu;         // expected resident workgroups per CU
  int pages_per_split;
  int n_splits;          // 1 (bf16 tokens) + ceil(max packed pages / pages_per_split)
};
bool decode_config(int heads, int n_sink, int n_recent, int batch, int max_seq_len, DecodeConfig* cfg);

}  // namespace mla
