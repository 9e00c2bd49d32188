/*
 * mla_lowbit.h - C ABI of the MI355X (gfx950) low-bit MLA KV-cache library.
 *
 * The library implements the decode hot path of QuantMLA's low-bit
 * Multi-Head Latent Attention cache (QuantMLA: Function-Aligned Dual-Path
 * Quantization for Low-Bit MLA KV Caching):
 *
 *  - every token's content latent c (d_c = 512) and decoupled RoPE key k_r
 *    (d_r = 64) are quantized per token, asymmetrically, in groups of 64
 *    channels, with one bf16 scale and one bf16 zero per group (ai.info
 *    summary, "Methodology in Plain English", last paragraph; onedev.kr
 *    review, "Premises and limits");
 *  - content codes are 4 or 2 bits, RoPE-key codes 4 bits (C4R4 / C2R4;
 *    ai.info summary, "Key Contributions", item 3);
 *  - a fused writer keeps a packed copy of every token plus the original
 *    bf16 rows of the first 4 ("sink") and the most recent 128 tokens
 *    (onedev.kr review, "How it is used"; ai.info summary, "Key
 *    Contributions", item 4);
 *  - decode attends over all valid tokens with one global softmax, each
 *    token entering exactly once: from its bf16 row when it is a sink or
 *    recent token, otherwise from its packed copy, unpacked and dequantized
 *    inside the attention loop (same sources).
 *
 * Conventions for every entry point
 *  - All buffer pointers are DEVICE pointers (HIP device memory), except the
 *    mla_lowbit_layout / mla_lowbit_cache structs themselves, which are read
 *    on the host during the call.  "bf16" buffers hold IEEE bfloat16 bit
 *    patterns (uint16).
 *  - The caller allocates and owns every buffer (cache, queries, outputs,
 *    workspace).  The library allocates no device memory and keeps no
 *    pointer after a call returns.
 *  - Calls are asynchronous and ordered on the given stream (hipStream_t
 *    passed as void*; NULL is the null stream).  An append must be issued
 *    before the decode that reads it, on the same stream (or with a
 *    dependency the caller creates).
 *  - Every entry point returns MLA_LOWBIT_OK or an error status, with a
 *    message in mla_lowbit_last_error() (thread-local).  Argument checks and
 *    kernel setup run on the host before anything is enqueued; a failure
 *    there enqueues nothing.  A decode enqueues three kernels (split plan,
 *    decode, combine); should a later launch fail after an earlier one was
 *    enqueued, the call returns MLA_LOWBIT_ERR_DEVICE with the HIP message and
 *    the enqueued kernels write the workspace and, of out and lse, only the
 *    rows of sequences decoded in one work item (see mla_lowbit_decode).
 *  - Device-resident index data (block_table entries, token positions,
 *    slots, sequence lengths) is the caller's contract.  The kernels never
 *    read or write outside the buffers the structs describe: an append skips
 *    a token whose page entry is out of range, a decode reads page 0 in place
 *    of an out-of-range page entry and treats a sequence with an out-of-range
 *    slot as empty; results for such inputs are wrong.  A decode counts these
 *    events in its workspace (and the bounded waits between the waves of the
 *    16-head kernel that gave up, which would mean a broken hand-over).
 *  - Validation mode: with the environment variable MLA_LOWBIT_VALIDATE set
 *    to a value other than "0" (read at every call), each call first
 *    synchronises the stream and checks the device-resident index data on
 *    the host (append: slots in range, 0 <= pos < slot_len_after[slot],
 *    distinct (slot, pos), written pages inside the table and the pool;
 *    decode: slots in range, 0 <= seq_len <= max_seq_len, every page read
 *    from packed copies inside the table and the pool; both: no physical page
 *    in the tables of two slots), returning MLA_LOWBIT_ERR_INVALID_ARG with
 *    the offending index before anything is enqueued.  After a decode it
 *    synchronises again and returns MLA_LOWBIT_ERR_DEVICE when the kernels
 *    counted any of the events above.  The mode is for debugging: it costs
 *    host copies of the index data and two stream synchronisations per call.
 *  - Value range.  Cache rows and queries must be finite with |x| < 65504
 *    (decode stages codes, bf16 rows, zeros and queries through fp16), and
 *    |sum over any 64-channel group of q| * softmax_scale < 45000.  Tested
 *    against the fp64 reference within the bounds below: caches scaled by
 *    1e-4 .. 300 (group scales from about 2^-15 to 2^13), and magnitudes
 *    growing by 3e5 along one sequence.  The PV products p * s are formed in
 *    fp16 with s normalised by a power of two per work item and group, so
 *    they neither overflow nor fall into subnormals over that range; values
 *    below 2^-14 in magnitude are carried as fp16 subnormals (absolute
 *    precision 2^-25).  Probabilities are fp16 (11 significant bits): when
 *    every score of a long sequence agrees to better than about 2^-11 (in
 *    log2 units; e.g. queries near zero against small cache values), the
 *    output is the near-uniform average without the finer weighting, an
 *    error up to 2^-11 of max |c| that can exceed the bound when max |out|
 *    is much smaller than max |c|.
 *  - Accuracy on the workloads' value distributions: max over channels of
 *    |out - ref| beyond half a bf16 ulp of ref, relative to max |ref| of the
 *    (sequence, head), <= 2e-3 against an fp64 reference of the same
 *    selected representations; |lse error| <= 1e-3 + 2^-18 |lse|.
 *
 * Supported layout: d_c = 512, d_r = 64, group = 64, page_tokens = 64,
 * bits_c in {4, 2}, bits_r = 4, 0 <= n_sink <= 64, 1 <= n_recent <= 2^24
 * (n_recent >= every sequence length gives an all-bf16 cache; long bf16
 * token lists are split over several work items like the packed pages).  num_heads
 * must be a positive multiple of 16.  Anything else returns
 * MLA_LOWBIT_ERR_UNSUPPORTED.
 */
#ifndef MLA_LOWBIT_H_
#define MLA_LOWBIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_LOWBIT_ABI_VERSION 1

enum {
  MLA_LOWBIT_OK = 0,
  MLA_LOWBIT_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad count */
  MLA_LOWBIT_ERR_UNSUPPORTED = 2, /* layout or head count this build does not implement */
  MLA_LOWBIT_ERR_WORKSPACE = 3,   /* workspace smaller than mla_lowbit_decode_workspace_bytes() */
  MLA_LOWBIT_ERR_DEVICE = 4       /* HIP launch / runtime error */
};

/* Shape and precision of the cache (mixed-precision policy included). */
typedef struct mla_lowbit_layout {
  int32_t abi_version; /* = MLA_LOWBIT_ABI_VERSION */
  int32_t d_c;         /* content latent width: 512 */
  int32_t d_r;         /* RoPE key width: 64 */
  int32_t bits_c;      /* content code bits: 4 (C4R4) or 2 (C2R4) */
  int32_t bits_r;      /* RoPE-key code bits: 4 */
  int32_t group;       /* channels per quantization group: 64 */
  int32_t page_tokens; /* tokens per cache page: 64 */
  int32_t n_sink;      /* leading tokens served from bf16: 4 */
  int32_t n_recent;    /* most recent tokens served from bf16: 128 */
} mla_lowbit_layout;

/*
 * The paged cache.  One page holds page_tokens consecutive tokens of one
 * sequence slot as three contiguous arrays (structure of arrays):
 *   [content codes: page_tokens x (d_c*bits_c/8) bytes]
 *   [RoPE-key codes: page_tokens x (d_r*bits_r/8) bytes]
 *   [metadata: page_tokens x 9 uint32]      (groups 0..7 content, 8 RoPE key)
 * Codes are packed low bits first in channel order (4-bit: byte k holds
 * channels 2k | 2k+1 << 4; 2-bit: byte k holds channels 4k .. 4k+3 at bit
 * offsets 0, 2, 4, 6).  A metadata dword holds bf16 scale s in bits 0..15 and
 * bf16 zero z in bits 16..31; a code q dequantizes to s*q + z.
 * Token t of slot i lives in page block_table[i*max_pages_per_seq + t/64],
 * row t%64.  Pages must be 256-byte aligned (the pool base must be).
 */
typedef struct mla_lowbit_cache {
  mla_lowbit_layout layout;
  void* pages;                /* [num_pages][page_bytes] */
  int64_t num_pages;
  void* sink;                 /* bf16 [num_slots][n_sink][d_c+d_r]; row i = token i */
  void* recent;               /* bf16 [num_slots][n_recent][d_c+d_r]; row p % n_recent = token p */
  int32_t num_slots;
  const int32_t* block_table; /* [num_slots][max_pages_per_seq] physical page ids */
  int32_t max_pages_per_seq;
} mla_lowbit_cache;

/* Bytes per cache page for this layout; 0 if the layout is unsupported. */
size_t mla_lowbit_page_bytes(const mla_lowbit_layout* layout);

/*
 * Fused quantize-append writer (onedev.kr review, "How it is used": the
 * writer keeps packed copies of all tokens and the bf16 values of the sink
 * and recent tokens).
 *
 * kv_new         bf16 [n_tokens][d_c+d_r], rows c || k_r (k_r after RoPE);
 *                16-byte aligned.
 * token_slot     int32 [n_tokens]: cache slot of each new token.
 * token_pos      int32 [n_tokens]: absolute position of the token in its
 *                sequence (0-based).
 * slot_len_after int32 [num_slots]: length of each slot once this call's
 *                tokens are in (only entries of slots named in token_slot
 *                are read).
 *
 * For every token: quantizes its 9 groups (per-token asymmetric affine,
 * group 64; scale s = bf16(fp32(max-min)/(2^b-1)), zero z = min, codes
 * rint_half_even((x-min)/s) clamped), packs codes and metadata into its page
 * row, copies the bf16 row into sink row pos when pos < n_sink, and into
 * recent row pos % n_recent when pos >= slot_len_after[slot] - n_recent.
 * A token that leaves the recent window is served from the packed copy
 * written here; nothing is re-quantized.  Tokens of one call must have
 * distinct (slot, pos).  n_tokens = 0 is a no-op.
 */
int mla_lowbit_quantize_append(const mla_lowbit_cache* cache, const void* kv_new, const int32_t* token_slot,
                               const int32_t* token_pos, const int32_t* slot_len_after, int32_t n_tokens,
                               void* stream);

/* Workspace bytes mla_lowbit_decode needs for this batch shape (0 on
 * unsupported arguments). */
size_t mla_lowbit_decode_workspace_bytes(const mla_lowbit_layout* layout, int32_t batch, int32_t num_heads,
                                         int32_t max_seq_len);

/*
 * Low-bit absorbed-MLA decode, one query token per sequence (ai.info
 * summary, "Key Contributions", item 4; onedev.kr review, "How it is used").
 *
 * q           bf16 [batch][num_heads][d_c+d_r] = absorbed q_c || q_r; 16-byte aligned.
 * seq_slot    int32 [batch]: cache slot of each sequence.
 * seq_len     int32 [batch]: valid tokens N of each sequence (0 <= N <= max_seq_len),
 *             counting the token appended for this step.
 * softmax_scale  fp32 scale applied to q_c.c + q_r.k_r.
 * out         bf16 [batch][num_heads][d_c]: softmax(scores) . c over the N
 *             tokens; N = 0 gives zeros.  16-byte aligned.
 * lse         fp32 [batch][num_heads] natural-log log-sum-exp of the scaled
 *             scores (-inf for N = 0); may be NULL.
 * workspace   device scratch of at least mla_lowbit_decode_workspace_bytes(),
 *             256-byte aligned; contents need no initialisation.
 *
 * Token t of a sequence is read from its bf16 row when t < n_sink or
 * t >= N - n_recent, otherwise from its packed copy.  The work is split
 * along the context into page-aligned chunks whose partial results are
 * merged exactly with a log-sum-exp combine.  A sequence decoded in one work
 * item (no packed tokens and at most one chunk of bf16 tokens, e.g. every
 * N <= n_sink + n_recent) has its out and lse rows written by the decode
 * kernel itself, with the combine's arithmetic, and skips the combine.
 */
int mla_lowbit_decode(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot, const int32_t* seq_len,
                      int32_t batch, int32_t num_heads, int32_t max_seq_len, float softmax_scale, void* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode of q_len query tokens per sequence at once (speculative / multi-token
 * prediction steps): every query shares one read of the cache, so the packed
 * bytes of a page serve q_len * num_heads rows.  Same computation as
 * mla_lowbit_decode for each query (ai.info summary, "Key Contributions",
 * item 4), with causal visibility: seq_len counts all q_len new tokens, and
 * query i (0-based) sees tokens t < seq_len - (q_len - 1 - i), each in the
 * representation the cache holds for it at length seq_len.
 *
 * q           bf16 [batch][q_len][num_heads][d_c+d_r]; 16-byte aligned.
 * out         bf16 [batch][q_len][num_heads][d_c]; a query that sees no token
 *             gives zeros.
 * lse         fp32 [batch][q_len][num_heads] (-inf for no visible token); may be NULL.
 * workspace   at least mla_lowbit_decode_workspace_bytes(layout, batch,
 *             q_len * num_heads, max_seq_len) bytes.
 * Other arguments as mla_lowbit_decode.  1 <= q_len <= n_recent + 1 (the
 * tokens a query does not see are then in the bf16 recent window), num_heads
 * a positive multiple of 16, q_len * num_heads <= 2^20; otherwise
 * MLA_LOWBIT_ERR_UNSUPPORTED.  q_len = 1 is mla_lowbit_decode.
 */
int mla_lowbit_decode_multi(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot,
                            const int32_t* seq_len, int32_t batch, int32_t q_len, int32_t num_heads,
                            int32_t max_seq_len, float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Decode without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments and results as mla_lowbit_decode, without
 * workspace / workspace_bytes: the library uses its built-in scratch, a
 * file-scope device array of MLA_LOWBIT_SCRATCH_BYTES (80 MiB) that every GPU
 * the library runs on holds until the process ends (its address is resolved
 * on the first call made with that device current).
 *  - Returns MLA_LOWBIT_ERR_WORKSPACE when mla_lowbit_decode_workspace_bytes()
 *    for this shape exceeds MLA_LOWBIT_SCRATCH_BYTES (e.g. 128 heads: up to
 *    64 sequences of any length; 16 heads: several hundred).
 *  - Allocates nothing and calls no allocating routine; the validation mode
 *    does not apply to it (the counters are still written to the scratch).
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last
 *    call's contents and needs no clearing (each call writes what it reads).
 *    Calls ordered on one stream are safe; calls that overlap on one GPU (on
 *    different streams, or from threads without ordering between them) race
 *    and give wrong results.
 */
#define MLA_LOWBIT_SCRATCH_BYTES ((size_t)80 << 20)
int mla_lowbit_decode_noalloc(const mla_lowbit_cache* cache, const void* q, const int32_t* seq_slot,
                              const int32_t* seq_len, int32_t batch, int32_t num_heads, int32_t max_seq_len,
                              float softmax_scale, void* out, float* lse, void* stream);

/*
 * Measurement aid (not needed for decoding).  Arms two caller-created HIP
 * events (hipEvent_t passed as void*) for the NEXT mla_lowbit_decode or
 * mla_lowbit_decode_multi call on this thread: that call records `start` on
 * its stream immediately before
 * the split-KV decode kernel and `stop` immediately after it (before the
 * log-sum-exp combine), so hipEventElapsedTime(start, stop) is that kernel's
 * duration.  The events are disarmed after that call (also when it fails).
 * Passing NULL, NULL disarms.  Returns MLA_LOWBIT_OK.
 */
int mla_lowbit_profile_decode_events(void* start, void* stop);

/* Static description of a status code. */
const char* mla_lowbit_status_string(int status);

/* Thread-local detail message of the last non-OK return on this thread. */
const char* mla_lowbit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LOWBIT_H_ */
