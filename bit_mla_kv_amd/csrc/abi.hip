// Host side of the C ABI declared in include/mla_lowbit.h: argument checks,
// status strings, the thread-local error message and the kernel launches.
// Nothing here allocates device memory.  Only the validation mode
// (MLA_LOWBIT_VALIDATE=1) synchronises the stream and copies index data and
// the decode counters to the host.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/mla_lowbit.h"
#include "mla_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_layout(const mla_lowbit_layout* L) {
  if (!L) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "layout is NULL");
  if (L->abi_version != MLA_LOWBIT_ABI_VERSION)
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "abi_version %d, library implements %d", L->abi_version,
                MLA_LOWBIT_ABI_VERSION);
  if (L->d_c != mla::kDc || L->d_r != mla::kDr || L->group != mla::kGroup || L->page_tokens != mla::kPageTokens)
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "layout (d_c=%d, d_r=%d, group=%d, page_tokens=%d) unsupported; "
                "need (512, 64, 64, 64)", L->d_c, L->d_r, L->group, L->page_tokens);
  if ((L->bits_c != 4 && L->bits_c != 2) || L->bits_r != 4)
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "bits (c=%d, r=%d) unsupported; need c in {4,2}, r = 4", L->bits_c,
                L->bits_r);
  if (L->n_sink < 0 || L->n_sink > 64 || L->n_recent < 1 || L->n_recent > (1 << 24))
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "n_sink=%d / n_recent=%d outside [0,64] / [1,2^24]", L->n_sink,
                L->n_recent);
  return MLA_LOWBIT_OK;
}

int check_cache(const mla_lowbit_cache* c) {
  if (!c) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "cache is NULL");
  int st = check_layout(&c->layout);
  if (st != MLA_LOWBIT_OK) return st;
  if (c->num_pages < 0 || c->num_slots < 0 || c->max_pages_per_seq < 0)
    return fail(MLA_LOWBIT_ERR_INVALID_ARG, "negative cache dimension");
  if (c->num_pages > 0 && (!c->pages || !aligned(c->pages, 256)))
    return fail(MLA_LOWBIT_ERR_INVALID_ARG, "pages must be a non-NULL 256-byte aligned device pointer");
  if (c->num_slots > 0) {
    if (!c->recent || !aligned(c->recent, 16))
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "recent must be a non-NULL 16-byte aligned device pointer");
    if (c->layout.n_sink > 0 && (!c->sink || !aligned(c->sink, 16)))
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "sink must be a non-NULL 16-byte aligned device pointer");
    if (c->max_pages_per_seq > 0 && !c->block_table)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "block_table is NULL");
  }
  return MLA_LOWBIT_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_LOWBIT_OK;
  return fail(MLA_LOWBIT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- validation mode
bool validate_mode() {
  const char* e = getenv("MLA_LOWBIT_VALIDATE");
  return e && e[0] && strcmp(e, "0") != 0;
}

int spin_limit() {
  const char* e = getenv("MLA_LOWBIT_SPIN_LIMIT");  // test knob: bound of a handshake wait
  if (!e || !e[0]) return mla::kDefaultSpin;
  const long v = strtol(e, nullptr, 10);
  return v < 0 ? 0 : (int)std::min<long>(v, mla::kDefaultSpin);
}

template <typename T>
hipError_t fetch(std::vector<T>& v, const void* dptr, size_t n) {
  v.resize(n);
  if (n == 0) return hipSuccess;
  return hipMemcpy(v.data(), dptr, n * sizeof(T), hipMemcpyDeviceToHost);
}

// The slot's pages [first, last] must be inside its table row and name pages of the pool, and no
// physical page may serve two slots.
int check_pages(const mla_lowbit_cache* c, const std::vector<int32_t>& bt, int slot, int64_t first, int64_t last,
                std::unordered_map<int32_t, int>& owner, const char* what) {
  for (int64_t i = first; i <= last; ++i) {
    if (i >= c->max_pages_per_seq)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: %s: slot %d needs page index %lld, max_pages_per_seq is %d",
                  what, slot, (long long)i, c->max_pages_per_seq);
    const int32_t pg = bt[(size_t)slot * c->max_pages_per_seq + i];
    if (pg < 0 || pg >= c->num_pages)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: %s: block_table[%d][%lld] = %d outside [0, %lld)", what, slot,
                  (long long)i, pg, (long long)c->num_pages);
    auto it = owner.emplace(pg, slot).first;
    if (it->second != slot)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: %s: page %d is in the tables of slots %d and %d", what, pg,
                  it->second, slot);
  }
  return MLA_LOWBIT_OK;
}

// Device-resident arguments of a decode: slots and lengths in range, and the pages every sequence
// reads from packed copies valid and unshared.
int validate_decode_inputs(const mla_lowbit_cache* c, const int32_t* seq_slot, const int32_t* seq_len, int batch,
                           int max_seq_len, hipStream_t s) {
  int st = device_status(hipStreamSynchronize(s), "validate: stream synchronize");
  if (st != MLA_LOWBIT_OK) return st;
  std::vector<int32_t> slots, lens, bt;
  if ((st = device_status(fetch(slots, seq_slot, batch), "validate: copy seq_slot")) != MLA_LOWBIT_OK) return st;
  if ((st = device_status(fetch(lens, seq_len, batch), "validate: copy seq_len")) != MLA_LOWBIT_OK) return st;
  if ((st = device_status(fetch(bt, c->block_table, (size_t)c->num_slots * c->max_pages_per_seq),
                          "validate: copy block_table")) != MLA_LOWBIT_OK)
    return st;
  std::unordered_map<int32_t, int> owner;
  for (int b = 0; b < batch; ++b) {
    if (slots[b] < 0 || slots[b] >= c->num_slots)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: seq_slot[%d] = %d outside [0, %d)", b, slots[b], c->num_slots);
    if (lens[b] < 0 || lens[b] > max_seq_len)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: seq_len[%d] = %d outside [0, max_seq_len = %d]", b, lens[b],
                  max_seq_len);
    const int64_t lo = c->layout.n_sink, hi = (int64_t)lens[b] - c->layout.n_recent;  // packed tokens [lo, hi)
    if (hi > lo && (st = check_pages(c, bt, slots[b], lo / mla::kPageTokens, (hi - 1) / mla::kPageTokens, owner,
                                     "decode")) != MLA_LOWBIT_OK)
      return st;
  }
  return MLA_LOWBIT_OK;
}

// Device-resident arguments of an append: slots, positions and lengths consistent, (slot, pos)
// pairs distinct, and every written page valid and unshared.
int validate_append_inputs(const mla_lowbit_cache* c, const int32_t* token_slot, const int32_t* token_pos,
                           const int32_t* slot_len_after, int n, hipStream_t s) {
  int st = device_status(hipStreamSynchronize(s), "validate: stream synchronize");
  if (st != MLA_LOWBIT_OK) return st;
  std::vector<int32_t> slots, pos, after, bt;
  if ((st = device_status(fetch(slots, token_slot, n), "validate: copy token_slot")) != MLA_LOWBIT_OK) return st;
  if ((st = device_status(fetch(pos, token_pos, n), "validate: copy token_pos")) != MLA_LOWBIT_OK) return st;
  if ((st = device_status(fetch(after, slot_len_after, c->num_slots), "validate: copy slot_len_after")) != MLA_LOWBIT_OK)
    return st;
  if ((st = device_status(fetch(bt, c->block_table, (size_t)c->num_slots * c->max_pages_per_seq),
                          "validate: copy block_table")) != MLA_LOWBIT_OK)
    return st;
  std::unordered_set<int64_t> seen;
  std::unordered_map<int32_t, int> owner;
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= c->num_slots)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: token_slot[%d] = %d outside [0, %d)", i, slots[i], c->num_slots);
    if (pos[i] < 0 || pos[i] >= after[slots[i]])
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: token_pos[%d] = %d outside [0, slot_len_after[%d] = %d)", i,
                  pos[i], slots[i], after[slots[i]]);
    if (!seen.insert(((int64_t)slots[i] << 32) | (uint32_t)pos[i]).second)
      return fail(MLA_LOWBIT_ERR_INVALID_ARG, "validate: (slot %d, pos %d) appears twice", slots[i], pos[i]);
    const int64_t pi = pos[i] / mla::kPageTokens;
    if ((st = check_pages(c, bt, slots[i], pi, pi, owner, "append")) != MLA_LOWBIT_OK) return st;
  }
  return MLA_LOWBIT_OK;
}

// After a decode in validation mode: the counters the kernels left in the workspace header.
int check_decode_counters(const int32_t* hdr_dev, hipStream_t s) {
  int st = device_status(hipStreamSynchronize(s), "validate: stream synchronize");
  if (st != MLA_LOWBIT_OK) return st;
  int32_t h[8];
  if ((st = device_status(hipMemcpy(h, hdr_dev, sizeof(h), hipMemcpyDeviceToHost), "validate: copy counters")) !=
      MLA_LOWBIT_OK)
    return st;
  if (h[mla::kHdrGiveUps] || h[mla::kHdrBadPages] || h[mla::kHdrBadSeqs] || h[mla::kHdrDropped])
    return fail(MLA_LOWBIT_ERR_DEVICE,
                "validate: decode results are unreliable: %d handshake wait(s) gave up, %d page read(s) with a "
                "block-table entry out of range, %d sequence(s) with a bad slot or length, %d work item(s) dropped",
                h[mla::kHdrGiveUps], h[mla::kHdrBadPages], h[mla::kHdrBadSeqs], h[mla::kHdrDropped]);
  return MLA_LOWBIT_OK;
}

struct WsLayout {
  size_t hdr_off, items_off, seq_off, ml_off, z_off, o_off, total;
};

WsLayout ws_layout(int batch, int heads, int max_items) {
  WsLayout w;
  const size_t rows = (size_t)max_items * heads;
  w.hdr_off = 0;
  w.items_off = 256;
  w.seq_off = w.items_off + align_up((size_t)max_items * 16, 256);
  w.ml_off = w.seq_off + align_up((size_t)batch * 16, 256);
  w.z_off = w.ml_off + align_up(rows * 2 * sizeof(float), 256);
  w.o_off = w.z_off + align_up(rows * 8 * sizeof(float), 256);
  w.total = w.o_off + rows * mla::kDc * sizeof(float);
  return w;
}

}  // namespace

// Built-in decode workspace of mla_lowbit_decode_noalloc: one copy on every GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is taken with hipGetSymbolAddress (per device, below) and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MLA_LOWBIT_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once resolved

// The scratch address on the current device, resolved on the first call made with that device
// current.
int scratch_on_current_device(void** out) {
  int dev = 0;
  int st = device_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != MLA_LOWBIT_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    st = device_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != MLA_LOWBIT_OK) return st;
    if (!ptr) return fail(MLA_LOWBIT_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_LOWBIT_OK;
}

}  // namespace

extern "C" {

size_t mla_lowbit_page_bytes(const mla_lowbit_layout* layout) {
  if (check_layout(layout) != MLA_LOWBIT_OK) return 0;
  return (size_t)mla::page_bytes(layout->bits_c);
}

int mla_lowbit_quantize_append(const mla_lowbit_cache* cache, const void* kv_new, const int32_t* token_slot,
                               const int32_t* token_pos, const int32_t* slot_len_after, int32_t n_tokens,
                               void* stream) {
  int st = check_cache(cache);
  if (st != MLA_LOWBIT_OK) return st;
  if (n_tokens < 0) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "n_tokens = %d < 0", n_tokens);
  if (n_tokens == 0) return MLA_LOWBIT_OK;
  if (!kv_new || !aligned(kv_new, 16)) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "kv_new must be 16-byte aligned");
  if (!token_slot || !token_pos || !slot_len_after)
    return fail(MLA_LOWBIT_ERR_INVALID_ARG, "token_slot, token_pos and slot_len_after must be non-NULL");
  if (cache->num_slots == 0) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "cache has no slots");
  mla::AppendParams p;
  p.pages = static_cast<uint8_t*>(cache->pages);
  p.num_pages = cache->num_pages;
  p.sink = static_cast<uint16_t*>(cache->sink);
  p.recent = static_cast<uint16_t*>(cache->recent);
  p.num_slots = cache->num_slots;
  p.block_table = cache->block_table;
  p.max_pages = cache->max_pages_per_seq;
  p.n_sink = cache->layout.n_sink;
  p.n_recent = cache->layout.n_recent;
  p.bits_c = cache->layout.bits_c;
  p.kv = static_cast<const uint16_t*>(kv_new);
  p.token_slot = token_slot;
  p.token_pos = token_pos;
  p.slot_len_after = slot_len_after;
  p.n_tokens = n_tokens;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_mode() &&
      (st = validate_append_inputs(cache, token_slot, token_pos, slot_len_after, n_tokens, s)) != MLA_LOWBIT_OK)
    return st;
  return device_status(mla::launch_append(p, s), "quantize_append launch");
}

size_t mla_lowbit_decode_workspace_bytes(const mla_lowbit_layout* layout, int32_t batch, int32_t num_heads,
                                         int32_t max_seq_len) {
  if (check_layout(layout) != MLA_LOWBIT_OK || batch < 0 || max_seq_len < 0) return 0;
  mla::DecodeConfig cfg;
  if (!mla::decode_config(num_heads, layout->n_sink, layout->n_recent, batch, max_seq_len, &cfg)) return 0;
  return ws_layout(batch, num_heads, cfg.max_items).total;
}

int mla_lowbit_profile_decode_events(void* start, void* stop) {
  g_prof_start = static_cast<hipEvent_t>(start);
  g_prof_stop = static_cast<hipEvent_t>(stop);
  return MLA_LOWBIT_OK;
}

static int decode_impl(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot, const int32_t* seq_len,
                       int32_t batch, int32_t q_len, int32_t heads_per_query, int32_t max_seq_len,
                       float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream, hipEvent_t ev0, hipEvent_t ev1, bool allow_validate = true) {
  int st = check_cache(cache);
  if (st != MLA_LOWBIT_OK) return st;
  if (batch < 0 || max_seq_len < 0)
    return fail(MLA_LOWBIT_ERR_INVALID_ARG, "batch=%d max_seq_len=%d must be >= 0", batch, max_seq_len);
  if (heads_per_query <= 0 || heads_per_query % 16 != 0)
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "num_heads=%d unsupported (a positive multiple of 16)",
                heads_per_query);
  if (q_len < 1 || q_len - 1 > cache->layout.n_recent || (int64_t)q_len * heads_per_query > (1 << 20))
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "q_len=%d unsupported (1 .. n_recent + 1 = %d, q_len * num_heads <= 2^20)",
                q_len, cache->layout.n_recent + 1);
  const int32_t num_heads = q_len * heads_per_query;  // rows per sequence
  mla::DecodeConfig cfg;
  if (!mla::decode_config(num_heads, cache->layout.n_sink, cache->layout.n_recent, batch, max_seq_len, &cfg))
    return fail(MLA_LOWBIT_ERR_UNSUPPORTED, "num_heads=%d unsupported (a positive multiple of 16)",
                num_heads);
  if (!std::isfinite(softmax_scale)) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (batch == 0) return MLA_LOWBIT_OK;
  if (!q || !aligned(q, 16)) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "q must be a 16-byte aligned device pointer");
  if (!out || !aligned(out, 16))
    return fail(MLA_LOWBIT_ERR_INVALID_ARG, "out must be a 16-byte aligned device pointer");
  if (!seq_slot || !seq_len) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "seq_slot and seq_len must be non-NULL");
  if (lse && !aligned(lse, 4)) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const WsLayout wl = ws_layout(batch, num_heads, cfg.max_items);
  if (!workspace || !aligned(workspace, 256))
    return fail(MLA_LOWBIT_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (workspace_bytes < wl.total)
    return fail(MLA_LOWBIT_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, wl.total);
  if (cache->num_slots == 0) return fail(MLA_LOWBIT_ERR_INVALID_ARG, "cache has no slots");

  mla::DecodeParams p;
  p.pages = static_cast<const uint8_t*>(cache->pages);
  p.num_pages = cache->num_pages;
  p.sink = static_cast<const uint16_t*>(cache->sink);
  p.recent = static_cast<const uint16_t*>(cache->recent);
  p.num_slots = cache->num_slots;
  p.block_table = cache->block_table;
  p.max_pages = cache->max_pages_per_seq;
  p.n_sink = cache->layout.n_sink;
  p.n_recent = cache->layout.n_recent;
  p.q = static_cast<const uint16_t*>(q);
  p.seq_slot = seq_slot;
  p.seq_len = seq_len;
  p.batch = batch;
  p.heads = num_heads;
  p.max_seq_len = max_seq_len;
  p.spin_limit = spin_limit();
  p.q_len = q_len;
  p.heads_per_query = heads_per_query;
  p.scale_log2e = (float)((double)softmax_scale * 1.4426950408889634);
  p.head_groups = num_heads / cfg.heads_per_wg;
  p.target_items = cfg.target_items;
  p.min_pages_per_split = cfg.min_pages_per_split;
  p.force_pages_per_split = cfg.force_pages_per_split;
  p.max_items = cfg.max_items;
  char* wsb = static_cast<char*>(workspace);
  p.plan_hdr = reinterpret_cast<int32_t*>(wsb + wl.hdr_off);
  p.items = reinterpret_cast<int32_t*>(wsb + wl.items_off);
  p.seq_info = reinterpret_cast<int32_t*>(wsb + wl.seq_off);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_off);
  p.ws_z = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.z_off);
  p.has_z = 1;  // the decode kernels leave the zero-term sums to the combine
  p.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.o_off);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool validate = allow_validate && validate_mode();
  if (validate && (st = validate_decode_inputs(cache, seq_slot, seq_len, batch, max_seq_len, s)) != MLA_LOWBIT_OK)
    return st;
  // everything a launch of this call can be refused for is checked before the first one
  if ((st = device_status(mla::prepare_decode(p, cache->layout.bits_c), "decode kernel setup")) != MLA_LOWBIT_OK)
    return st;
  st = device_status(mla::launch_plan(p, s), "plan launch");
  if (st != MLA_LOWBIT_OK) return st;
  if (ev0 && (st = device_status(hipEventRecord(ev0, s), "profile start event")) != MLA_LOWBIT_OK) return st;
  st = device_status(mla::launch_decode(p, cache->layout.bits_c, s), "decode launch");
  if (st != MLA_LOWBIT_OK) return st;
  if (ev1 && (st = device_status(hipEventRecord(ev1, s), "profile stop event")) != MLA_LOWBIT_OK) return st;
  st = device_status(mla::launch_combine(p, s), "combine launch");
  if (st != MLA_LOWBIT_OK || !validate) return st;
  return check_decode_counters(p.plan_hdr, s);
}

int mla_lowbit_decode(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot, const int32_t* seq_len,
                      int32_t batch, int32_t num_heads, int32_t max_seq_len, float softmax_scale, void* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  return decode_impl(cache, q, seq_slot, seq_len, batch, 1, num_heads, max_seq_len, softmax_scale, out, lse,
                     workspace, workspace_bytes, stream, ev0, ev1);
}

int mla_lowbit_decode_multi(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot,
                            const int32_t* seq_len, int32_t batch, int32_t q_len, int32_t num_heads,
                            int32_t max_seq_len, float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  return decode_impl(cache, q, seq_slot, seq_len, batch, q_len, num_heads, max_seq_len, softmax_scale, out, lse,
                     workspace, workspace_bytes, stream, ev0, ev1);
}

int mla_lowbit_decode_noalloc(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot,
                              const int32_t* seq_len, int32_t batch, int32_t num_heads, int32_t max_seq_len,
                              float softmax_scale, void* out, float* lse, void* stream) {
  hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  int st = check_cache(cache);
  if (st != MLA_LOWBIT_OK) return st;
  const size_t need = mla_lowbit_decode_workspace_bytes(&cache->layout, batch, num_heads, max_seq_len);
  if (need > MLA_LOWBIT_SCRATCH_BYTES)
    return fail(MLA_LOWBIT_ERR_WORKSPACE, "this shape needs %zu workspace bytes; the built-in scratch holds %zu",
                need, (size_t)MLA_LOWBIT_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != MLA_LOWBIT_OK) return st;
  return decode_impl(cache, q, seq_slot, seq_len, batch, 1, num_heads, max_seq_len, softmax_scale, out, lse, ws,
                     MLA_LOWBIT_SCRATCH_BYTES, stream, ev0, ev1, /*allow_validate=*/false);
}

}  // extern "C"

extern "C" {

const char* mla_lowbit_status_string(int status) {
  switch (status) {
    case MLA_LOWBIT_OK: return "ok";
    case MLA_LOWBIT_ERR_INVALID_ARG: return "invalid argument";
    case MLA_LOWBIT_ERR_UNSUPPORTED: return "unsupported layout or shape";
    case MLA_LOWBIT_ERR_WORKSPACE: return "workspace too small";
    case MLA_LOWBIT_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* mla_lowbit_last_error(void) { return g_err; }

}  // extern "C"
