/*
 * oracle.c -- plain, slow, single-threaded CPU reference for paged decode
 * attention and the two KV-cache write paths.  TEST INFRASTRUCTURE ONLY:
 * it is loaded by the tests, by the smoke check and by the benchmark's CPU
 * baseline leg, never by the library.  It shares no code, header or table
 * with the HIP path.
 *
 * What it follows:
 *  - Pool of fixed-size blocks, each holding block_size tokens of one layer's
 *    K (or V) for every KV head; a per-sequence block table maps logical block
 *    i to a physical block anywhere in the pool.  Page "vLLM 与 KV Cache",
 *    virtual-memory table and how-it-works points 1-2; page "vLLM KV Cache
 *    实现机制" §1.2 diagram and §4.1 pool diagram; page "vLLM — 把操作系统的分页
 *    搬进 GPU KV cache", core mechanisms (fixed blocks, indirection).
 *  - Decode reads K/V by looking up the table for the physical block and then
 *    offsetting into it: same page 3, core mechanisms, kernel paragraph.
 *  - Attention of one new query token over every cached token (page 1, why a
 *    KV cache), computed here as textbook softmax(q K^T * scale) V in fp64
 *    after first materialising the sequence's contiguous K/V.
 *  - Copy-on-write of a shared block (page 3, core mechanism 3 and case 2).
 *
 * Pool layout (the format the library exports; both sides must agree on it
 * byte for byte): element (block b, kv head h, token slot o, dim j) of a pool
 * with H kv heads, block size B and head dim D sits at element index
 * ((b*H + h)*B + o)*D + j.
 *
 * Number formats are decoded from their definitions: IEEE binary16, bfloat16
 * (the upper half of an IEEE binary32), and OCP 8-bit E4M3 "FN" (bias 7, no
 * infinities, S.1111.111 is NaN, largest finite 448).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8E4M3 = 3 };
enum { OR_OK = 0, OR_BAD_ARG = 1, OR_BAD_LEN = 2, OR_BAD_BLOCK = 3, OR_NOMEM = 4 };

static size_t elem_bytes(int dt) {
  switch (dt) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    case OR_FP8E4M3: return 1;
  }
  return 0;
}

/* ---------------------------------------------------------------- decoders */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);            /* subnormal: m * 2^-10 * 2^-14 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 0xff, m = b & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133);            /* m * 2^-7 * 2^-126 */
  else if (e == 255)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent field 15
 * with fraction 7 is NaN, every other pattern is finite. */
double oracle_e4m3_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
  else
    v = ldexp((double)(8 + m), e - 10);    /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

static double load_elem(const void* base, int dt, size_t idx) {
  switch (dt) {
    case OR_F32: {
      float f;
      memcpy(&f, (const char*)base + 4 * idx, 4);
      return (double)f;
    }
    case OR_F16: {
      uint16_t h;
      memcpy(&h, (const char*)base + 2 * idx, 2);
      return oracle_f16_to_f64(h);
    }
    case OR_BF16: {
      uint16_t b;
      memcpy(&b, (const char*)base + 2 * idx, 2);
      return oracle_bf16_to_f64(b);
    }
    case OR_FP8E4M3:
      return oracle_e4m3_to_f64(((const uint8_t*)base)[idx]);
  }
  return NAN;
}

/* ---------------------------------------------------------------- encoder */

/* Magnitudes of the 127 non-negative finite E4M3FN codes 0x00..0x7E, which
 * increase with the code. */
static double e4m3_mag[127];
static int e4m3_ready = 0;

static void e4m3_init(void) {
  if (e4m3_ready) return;
  for (int c = 0; c < 127; ++c) e4m3_mag[c] = oracle_e4m3_to_f64((uint8_t)c);
  e4m3_ready = 1;
}

/* Nearest E4M3FN value to x, ties to the even code (round-to-nearest-even on
 * the fraction), saturating finite overflow to +-448; NaN maps to 0x7F. */
uint8_t oracle_f32_to_e4m3_sat(float xf) {
  e4m3_init();
  if (isnan(xf)) return 0x7F;
  double x = (double)xf;
  uint8_t sign = signbit(xf) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a >= e4m3_mag[126]) return sign | 126;
  /* largest code with magnitude <= a */
  int lo = 0, hi = 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (e4m3_mag[mid] <= a) lo = mid; else hi = mid;
  }
  double dlo = a - e4m3_mag[lo], dhi = e4m3_mag[hi] - a;
  int c;
  if (dlo < dhi) c = lo;
  else if (dhi < dlo) c = hi;
  else c = (lo % 2 == 0) ? lo : hi;
  return sign | (uint8_t)c;
}

/* ------------------------------------------------------- cache write paths */

/* Value of a source element as fp32 (exact for f32/f16/bf16 sources). */
static float src_as_f32(const void* base, int dt, size_t idx) {
  return (float)load_elem(base, dt, idx);
}

/*
 * Write the K/V of T tokens into their slots.  Slot s means token offset
 * s mod B of physical block floor(s / B).  A negative slot skips the token.
 * Same source and pool dtype: bytes are copied.  fp8 pool: each element is
 * encoded as E4M3FN of (fp32(x) / fp32(scale)), where scale is the tensor's
 * scale, or head h's scale when k_head / v_head ([H] each) are given.
 * k, v: [T][H][D] in src_dtype.
 */
int oracle_reshape_and_cache(void* kpool, void* vpool, int pool_dtype, int64_t num_blocks, int B, int H, int D,
                             float k_scale, float v_scale, const void* k, const void* v, int src_dtype,
                             const int64_t* slots, int64_t T, const float* k_head, const float* v_head) {
  if (!kpool || !vpool || !k || !v || !slots || B <= 0 || H <= 0 || D <= 0) return OR_BAD_ARG;
  int quant = pool_dtype == OR_FP8E4M3 && src_dtype != OR_FP8E4M3;
  if (!quant && src_dtype != pool_dtype) return OR_BAD_ARG;
  size_t eb = elem_bytes(pool_dtype), sb = elem_bytes(src_dtype);
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slots[t];
    if (s < 0) continue;
    int64_t b = s / B, o = s % B;
    if (b >= num_blocks) return OR_BAD_BLOCK;
    for (int h = 0; h < H; ++h) {
      size_t dst = ((size_t)(b * H + h) * B + o) * D;
      size_t src = ((size_t)t * H + h) * D;
      if (!quant) {
        memcpy((char*)kpool + dst * eb, (const char*)k + src * sb, D * eb);
        memcpy((char*)vpool + dst * eb, (const char*)v + src * sb, D * eb);
      } else {
        const float ks = k_head ? k_head[h] : k_scale, vs = v_head ? v_head[h] : v_scale;
        for (int j = 0; j < D; ++j) {
          float xk = src_as_f32(k, src_dtype, src + j) / ks;
          float xv = src_as_f32(v, src_dtype, src + j) / vs;
          ((uint8_t*)kpool)[dst + j] = oracle_f32_to_e4m3_sat(xk);
          ((uint8_t*)vpool)[dst + j] = oracle_f32_to_e4m3_sat(xv);
        }
      }
    }
  }
  return OR_OK;
}

/* Copy whole physical blocks (every head and every slot) src -> dst, for each
 * (src, dst) pair.  block_bytes = H * B * D * elem bytes of one pool. */
int oracle_copy_blocks(void* kpool, void* vpool, int64_t block_bytes, int64_t num_blocks, const int32_t* pairs,
                       int64_t P) {
  if (!kpool || !vpool || (P > 0 && !pairs)) return OR_BAD_ARG;
  for (int64_t i = 0; i < P; ++i) {
    int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || d < 0 || s >= num_blocks || d >= num_blocks) return OR_BAD_BLOCK;
    memcpy((char*)kpool + d * block_bytes, (const char*)kpool + s * block_bytes, (size_t)block_bytes);
    memcpy((char*)vpool + d * block_bytes, (const char*)vpool + s * block_bytes, (size_t)block_bytes);
  }
  return OR_OK;
}

/* Move whole blocks between the pool and a host swap area (offload / SWAP
 * preemption: page "vLLM KV Cache 实现机制" §2.1 storage tiers; page "vLLM —
 * 把操作系统的分页搬进 GPU KV cache", case 3).  out != 0: pool block src ->
 * host block dst; out == 0: host block src -> pool block dst.  Ids out of
 * range are an error here (the oracle is strict). */
int oracle_swap_blocks(void* kpool, void* vpool, int64_t num_blocks, void* khost, void* vhost, int64_t host_blocks,
                       int64_t block_bytes, const int32_t* pairs, int64_t P, int out) {
  if (!kpool || !vpool || !khost || !vhost || (P > 0 && !pairs)) return OR_BAD_ARG;
  for (int64_t i = 0; i < P; ++i) {
    int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    int64_t sn = out ? num_blocks : host_blocks, dn = out ? host_blocks : num_blocks;
    if (s < 0 || d < 0 || s >= sn || d >= dn) return OR_BAD_BLOCK;
    char* sk = (char*)(out ? kpool : khost) + s * block_bytes;
    char* sv = (char*)(out ? vpool : vhost) + s * block_bytes;
    char* dk = (char*)(out ? khost : kpool) + d * block_bytes;
    char* dv = (char*)(out ? vhost : vpool) + d * block_bytes;
    memcpy(dk, sk, (size_t)block_bytes);
    memcpy(dv, sv, (size_t)block_bytes);
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ decode */

/* Contiguous K and V (fp64, dequantised) of the first n tokens of sequence s,
 * KV head hk: token t lives at slot t % B of block block_tables[s][t / B].
 * fp8 codes are multiplied by the tensor's scale, or head hk's scale when
 * k_head / v_head are given. */
static int materialise_kv(const void* kpool, const void* vpool, int kv_dtype, int64_t num_blocks, int B, int H,
                          int D, double k_scale, double v_scale, const float* k_head, const float* v_head,
                          const int32_t* block_tables, int max_blocks, int s, int hk, int n, double* Kc, double* Vc) {
  int fp8 = kv_dtype == OR_FP8E4M3;
  if (k_head) k_scale = k_head[hk];
  if (v_head) v_scale = v_head[hk];
  for (int t = 0; t < n; ++t) {
    int32_t blk = block_tables[(size_t)s * max_blocks + t / B];
    int o = t % B;
    if (blk < 0 || blk >= num_blocks) return OR_BAD_BLOCK;
    size_t base = ((size_t)((int64_t)blk * H + hk) * B + o) * D;
    for (int j = 0; j < D; ++j) {
      double kv = load_elem(kpool, kv_dtype, base + j);
      double vv = load_elem(vpool, kv_dtype, base + j);
      Kc[(size_t)t * D + j] = fp8 ? kv * k_scale : kv;
      Vc[(size_t)t * D + j] = fp8 ? vv * v_scale : vv;
    }
  }
  return OR_OK;
}

/* Textbook softmax attention of one query row qd over tokens 0..nt-1:
 * score_t = scale * <qd, Kc[t]>, m = max score, p_t = exp(score_t - m),
 * l = sum p_t, o = sum_t p_t Vc[t] / l.  sc is scratch of nt doubles. */
static void attend(const double* qd, const double* Kc, const double* Vc, int nt, int D, double scale, double* sc,
                   double* o) {
  double m = -INFINITY;
  for (int t = 0; t < nt; ++t) {
    double acc = 0.0;
    for (int j = 0; j < D; ++j) acc += qd[j] * Kc[(size_t)t * D + j];
    sc[t] = scale * acc;
    if (sc[t] > m) m = sc[t];
  }
  double l = 0.0;
  for (int t = 0; t < nt; ++t) {
    sc[t] = exp(sc[t] - m);
    l += sc[t];
  }
  for (int j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int t = 0; t < nt; ++t) acc += sc[t] * Vc[(size_t)t * D + j];
    o[j] = acc / l;
  }
}

/*
 * out[s][hq][:] (fp64) for every sequence s listed in `seqs` (all when seqs
 * is NULL):
 *   n = context_lens[s]  (1 <= n <= max_blocks * B)
 *   for token t < n: blk = block_tables[s][t / B], o = t % B,
 *     Kc[t][:] = K[blk][hkv][o][:] * k_scale (fp8 pools only; the scale of
 *     kv head hkv when k_head / v_head are given), same for V,
 *     where hkv = hq / (Hq / H)
 *   score_t = scale * sum_j q[s][hq][j] * Kc[t][j]
 *   m = max_t score_t, p_t = exp(score_t - m), l = sum_t p_t
 *   out = sum_t p_t * Vc[t] / l
 */
int oracle_decode(const void* kpool, const void* vpool, int kv_dtype, int64_t num_blocks, int B, int H, int D,
                  double k_scale, double v_scale, const void* q, int q_dtype, int S, int Hq,
                  const int32_t* block_tables, int max_blocks, const int32_t* context_lens, double scale,
                  const int32_t* seqs, int n_seqs, double* out, const float* k_head, const float* v_head) {
  if (!kpool || !vpool || !q || !block_tables || !context_lens || !out) return OR_BAD_ARG;
  if (B <= 0 || H <= 0 || D <= 0 || Hq <= 0 || Hq % H != 0 || max_blocks <= 0) return OR_BAD_ARG;
  int g = Hq / H;
  int count = seqs ? n_seqs : S;
  for (int si = 0; si < count; ++si) {
    int s = seqs ? seqs[si] : si;
    if (s < 0 || s >= S) return OR_BAD_ARG;
    int n = context_lens[s];
    if (n < 1 || (int64_t)n > (int64_t)max_blocks * B) return OR_BAD_LEN;
    double* Kc = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* sc = (double*)malloc(sizeof(double) * (size_t)n);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    int rc = (Kc && Vc && sc && qd) ? OR_OK : OR_NOMEM;
    for (int hk = 0; hk < H && rc == OR_OK; ++hk) {
      rc = materialise_kv(kpool, vpool, kv_dtype, num_blocks, B, H, D, k_scale, v_scale, k_head, v_head,
                          block_tables, max_blocks, s, hk, n, Kc, Vc);
      for (int gi = 0; gi < g && rc == OR_OK; ++gi) {
        int hq = hk * g + gi;
        size_t qoff = ((size_t)s * Hq + hq) * D;
        for (int j = 0; j < D; ++j) qd[j] = load_elem(q, q_dtype, qoff + j);
        attend(qd, Kc, Vc, n, D, scale, sc, out + qoff);
      }
    }
    free(Kc);
    free(Vc);
    free(sc);
    free(qd);
    if (rc != OR_OK) return rc;
  }
  return OR_OK;
}

/*
 * Several new query tokens per sequence attending causally to the paged
 * context (chunked prefill / verification of speculative tokens).  Sequence
 * s owns query rows [query_start[s], query_start[s+1]); its m new tokens are
 * the last m of its n = context_lens[s] cached tokens, so query row i sits at
 * position n - m + (i - query_start[s]) and attends to tokens 0..position.
 * Per (row, query head) the result is the decode formula above restricted to
 * those tokens.  q and out are [total_q][Hq][D]; out is fp64.
 */
int oracle_prefill(const void* kpool, const void* vpool, int kv_dtype, int64_t num_blocks, int B, int H, int D,
                   double k_scale, double v_scale, const void* q, int q_dtype, int S, int Hq,
                   const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                   const int32_t* query_start, double scale, double* out, const float* k_head,
                   const float* v_head) {
  if (!kpool || !vpool || !q || !block_tables || !context_lens || !query_start || !out) return OR_BAD_ARG;
  if (B <= 0 || H <= 0 || D <= 0 || Hq <= 0 || Hq % H != 0 || max_blocks <= 0) return OR_BAD_ARG;
  int g = Hq / H;
  for (int s = 0; s < S; ++s) {
    int n = context_lens[s];
    int q0 = query_start[s], m = query_start[s + 1] - q0;
    if (m < 0 || m > n || n < 1 || (int64_t)n > (int64_t)max_blocks * B) return OR_BAD_LEN;
    if (m == 0) continue;
    double* Kc = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)n * D);
    double* sc = (double*)malloc(sizeof(double) * (size_t)n);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    int rc = (Kc && Vc && sc && qd) ? OR_OK : OR_NOMEM;
    for (int hk = 0; hk < H && rc == OR_OK; ++hk) {
      rc = materialise_kv(kpool, vpool, kv_dtype, num_blocks, B, H, D, k_scale, v_scale, k_head, v_head,
                          block_tables, max_blocks, s, hk, n, Kc, Vc);
      for (int i = 0; i < m && rc == OR_OK; ++i) {
        int seen = n - m + i + 1;
        for (int gi = 0; gi < g; ++gi) {
          int hq = hk * g + gi;
          size_t qoff = ((size_t)(q0 + i) * Hq + hq) * D;
          for (int j = 0; j < D; ++j) qd[j] = load_elem(q, q_dtype, qoff + j);
          attend(qd, Kc, Vc, seen, D, scale, sc, out + qoff);
        }
      }
    }
    free(Kc);
    free(Vc);
    free(sc);
    free(qd);
    if (rc != OR_OK) return rc;
  }
  return OR_OK;
}

/* KV-cache footprint in bytes: 2 (K and V) * layers * heads * head_dim *
 * tokens * bytes per element.  Page "vLLM 与 KV Cache", memory problem
 * equation; page "vLLM KV Cache 实现机制", §2.2 formula. */
double oracle_kv_footprint_bytes(int layers, int heads, int head_dim, int64_t tokens, int dtype_bytes) {
  return 2.0 * layers * heads * head_dim * (double)tokens * dtype_bytes;
}
