/*
 * CPU oracle for the low-bit MLA decode path.  TEST INFRASTRUCTURE ONLY:
 * only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load it.  It shares no code, header or table with the HIP library.
 *
 * What it computes, step by step, in the order the QuantMLA pages give it:
 *
 *  1. Per-token asymmetric affine quantization with group size 64 (ai.info
 *     summary, "Methodology in Plain English", last paragraph; onedev.kr
 *     review, "Premises and limits"): every token, including the protected
 *     sink and recent ones, gets a packed copy (onedev.kr review, "How it is
 *     used").  Content groups use bits_c in {4, 2}, the RoPE-key group 4 bits
 *     (C4R4 / C2R4; ai.info summary, "Key Contributions", item 3).
 *     The pages do not fix the arithmetic; the reading used here is
 *       mn = min x, mx = max x
 *       s  = bf16_rne(fp32(fp32(mx - mn) / Lb)),   Lb = 2^b - 1
 *       z  = mn (exact in bf16; -0 stored as +0)
 *       q  = 0 if s == 0 else clamp(rint_half_even(fp32(fp32(x - mn) / s)), 0, Lb)
 *       dequantized value = s * q + z   (evaluated in fp64, exact)
 *     There is no a*b+c anywhere, so FMA contraction cannot change it; the
 *     file is still built with -ffp-contract=off.
 *  2. Packing: low bits first, channels in order; metadata per group is one
 *     dword (bf16 s in the low half, bf16 z in the high half).
 *  3. Selection: token t of a sequence of N tokens uses its original bf16 row
 *     when t < n_sink or t >= N - n_recent, and its dequantized packed copy
 *     otherwise, so every valid token has exactly one representation
 *     (onedev.kr review, "How it is used"; ai.info summary, "Key
 *     Contributions", item 4: first 4 sink tokens, most recent 128 tokens).
 *  4. Exact absorbed-MLA attention in fp64 over all N tokens with one global
 *     softmax: sigma_t = scale * (q_c . c_t + q_r . k_r,t), output
 *     sum_t softmax(sigma)_t * c_t (the content latent is both matched and
 *     aggregated; onedev.kr review, "How it differs"), lse = m + ln(l).
 *
 * Parity of the quantizer arithmetic with the pages is unpinnable (the pages
 * print no worked example); it is pinned by hand-derived examples, the
 * s/2 round-trip bound and brute force in tests/.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MLO_DC 512
#define MLO_DR 64
#define MLO_D (MLO_DC + MLO_DR)
#define MLO_G 64

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Quantize one group of 64 bf16 values to codes (one per byte, unpacked). */
static void quantize_group(const uint16_t* x, int bits, uint8_t* q, uint16_t* s_bits, uint16_t* z_bits) {
  float mn = bf16_to_f32(x[0]), mx = mn;
  for (int i = 1; i < MLO_G; ++i) {
    float v = bf16_to_f32(x[i]);
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  const int lb = (1 << bits) - 1;
  float range = mx - mn;
  float s32 = range / (float)lb;
  uint16_t sb = f32_to_bf16_rne(s32);
  float s = bf16_to_f32(sb);
  uint16_t zb = f32_to_bf16_rne(mn);
  if (zb == 0x8000u) zb = 0; /* -0 -> +0 */
  for (int i = 0; i < MLO_G; ++i) {
    if (s == 0.0f) {
      q[i] = 0;
      continue;
    }
    float d = (bf16_to_f32(x[i]) - mn) / s;
    float r = rintf(d); /* default rounding mode: nearest, ties to even */
    int c = (int)r;
    if (c < 0) c = 0;
    if (c > lb) c = lb;
    q[i] = (uint8_t)c;
  }
  *s_bits = sb;
  *z_bits = zb;
}

static void pack(const uint8_t* q, int n, int bits, uint8_t* out) {
  int per = 8 / bits;
  for (int k = 0; k < n / per; ++k) {
    unsigned b = 0;
    for (int j = 0; j < per; ++j) b |= (unsigned)q[k * per + j] << (j * bits);
    out[k] = (uint8_t)b;
  }
}

static int unpack_one(const uint8_t* packed, int i, int bits) {
  int per = 8 / bits;
  return (packed[i / per] >> ((i % per) * bits)) & ((1 << bits) - 1);
}

/* Quantize + pack n tokens.  rows: [n][576] bf16 (c || k_r).
 * codes_c: [n][512*bits_c/8], codes_r: [n][64*4/8], meta: [n][9]. */
void mlo_quantize_tokens(const uint16_t* rows, int64_t n, int bits_c, uint8_t* codes_c, uint8_t* codes_r,
                         uint32_t* meta) {
  const int cb = MLO_DC * bits_c / 8;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    const uint16_t* x = rows + t * MLO_D;
    uint8_t q[MLO_D];
    for (int g = 0; g < 9; ++g) {
      int bits = g < 8 ? bits_c : 4;
      uint16_t sb, zb;
      quantize_group(x + g * MLO_G, bits, q + g * MLO_G, &sb, &zb);
      meta[t * 9 + g] = (uint32_t)sb | ((uint32_t)zb << 16);
    }
    pack(q, MLO_DC, bits_c, codes_c + t * cb);
    pack(q + MLO_DC, MLO_DR, 4, codes_r + t * (MLO_DR / 2));
  }
}

/* Selected representation of every token of one sequence (fp64). */
void mlo_select(const uint16_t* rows, const uint8_t* codes_c, const uint8_t* codes_r, const uint32_t* meta,
                int64_t n, int bits_c, int n_sink, int n_recent, double* sel) {
  const int cb = MLO_DC * bits_c / 8;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    double* o = sel + t * MLO_D;
    if (t < n_sink || t >= n - n_recent) {
      for (int i = 0; i < MLO_D; ++i) o[i] = (double)bf16_to_f32(rows[t * MLO_D + i]);
      continue;
    }
    for (int i = 0; i < MLO_D; ++i) {
      int g = i / MLO_G;
      uint32_t md = meta[t * 9 + g];
      double s = (double)bf16_to_f32((uint16_t)(md & 0xFFFFu));
      double z = (double)bf16_to_f32((uint16_t)(md >> 16));
      int c = i < MLO_DC ? unpack_one(codes_c + t * cb, i, bits_c)
                         : unpack_one(codes_r + t * (MLO_DR / 2), i - MLO_DC, 4);
      o[i] = s * (double)c + z;
    }
  }
}

/* Exact attention for the listed heads over selected rows sel [n][576].
 * q: [H][576] bf16.  out: [n_heads][512], lse: [n_heads] (natural log). */
void mlo_attend(const double* sel, int64_t n, const uint16_t* q, const int32_t* heads, int n_heads, double scale,
                double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < n_heads; ++j) {
    double qd[MLO_D];
    for (int i = 0; i < MLO_D; ++i) qd[i] = (double)bf16_to_f32(q[(int64_t)heads[j] * MLO_D + i]);
    double* o = out + (int64_t)j * MLO_DC;
    for (int i = 0; i < MLO_DC; ++i) o[i] = 0.0;
    if (n == 0) {
      lse[j] = -INFINITY;
      continue;
    }
    double* sc = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      const double* k = sel + t * MLO_D;
      double acc = 0.0;
      for (int i = 0; i < MLO_D; ++i) acc += qd[i] * k[i];
      sc[t] = scale * acc;
      if (sc[t] > m) m = sc[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      double w = exp(sc[t] - m);
      l += w;
      const double* k = sel + t * MLO_D;
      for (int i = 0; i < MLO_DC; ++i) o[i] += w * k[i];
    }
    for (int i = 0; i < MLO_DC; ++i) o[i] /= l;
    lse[j] = m + log(l);
    free(sc);
  }
}

int mlo_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
