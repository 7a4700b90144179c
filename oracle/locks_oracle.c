/*
 * locks_oracle.c — plain, slow fp64 CPU oracle of the LOCKS decode path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product (the HIP library and its
 * Python binding) includes, links, loads or calls this file; only the tests,
 * the smoke check and the benchmark's CPU-baseline leg do. It shares no code,
 * header, table or constant with the GPU path: the record format below is
 * re-derived here from its documented definition.
 *
 * Sources (cited by title and section):
 *   (A) "LOCKS: per-page SVD cuts KV-cache reads 10x at 1M context" — sections
 *       "How LOCKS works" (summary contents, page-score equation), "Code"
 *       (build loop, scoring loop, top-k, attention), "Caveats".
 *   (B) "LOCKS – 효율적인 롱 컨텍스트 디코딩을 위한 페이지 로컬 압축 키 요약"
 *       (gist.science, paper 2607.24555) — section 2, mechanism 1 (page-local
 *       eigendecomposition, int4 basis, int8 coefficients and centroid, r = 8,
 *       page size 16), mechanism 2 (reconstructed in-page logits and their
 *       log-sum-exp), mechanism 3 (GQA group-shared selection).
 *
 * All arithmetic is double precision on the exact input bits (bf16 keys and
 * values, fp32 queries). Each step is written in the order the pages give it;
 * the only library routines are libm's exp/log/sqrt/rint and qsort.
 * OpenMP only spreads independent (page, head) or (sequence, KV head) units
 * over threads; it changes no arithmetic.
 *
 * Readings of points the pages leave open (each is listed in the design
 * notes): one fp16 absmax scale per tensor per page; symmetric ranges +-127
 * (int8) and +-7 (int4), round half to even; coefficients taken from the
 * unquantised basis; Jacobi on the 16x16 Gram of the centred keys; group key =
 * log of the group-mean normalised mass share; top-k ties to the lower page
 * id; ids output ascending; the tokens of the last, partly filled page (no
 * summary yet: summaries are built when a page fills) are always attended.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OD 128        /* head dimension */
#define OP 16         /* tokens per page */
#define OR 8          /* rank of the shipped summary */
#define OSTRIDE 784   /* bytes per summary record */
#define OV_OFF 0      /* V codes */
#define OMU_OFF 512   /* centroid codes */
#define OC_OFF 640    /* coefficient codes */
#define OS_OFF 768    /* fp16 scales */

/* ------------------------------------------------------------------ */
/* Number formats                                                       */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction bits). */
double oracle_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even; returns the bits. */
uint16_t oracle_double_to_f16(double x) {
  uint16_t sign = 0;
  if (x < 0 || (x == 0 && signbit(x))) { sign = 0x8000; x = -x; }
  if (isnan(x)) return 0x7e00;
  if (x == 0) return sign;
  /* 65520 = largest finite (65504) plus half its spacing: ties go to even = inf */
  if (x >= 65520.0) return sign | 0x7c00;
  int e2;
  frexp(x, &e2);                  /* x = f * 2^e2, f in [0.5, 1) -> binade 2^(e2-1) */
  int e = e2 - 1;                 /* x in [2^e, 2^(e+1)) */
  double quantum = (e < -14) ? ldexp(1.0, -24) : ldexp(1.0, e - 10);
  double n = rint(x / quantum);   /* exact division by a power of two; ties to even */
  double v = n * quantum;
  if (v >= 65520.0) return sign | 0x7c00;
  if (v < ldexp(1.0, -14)) {      /* subnormal (or rounded up to the smallest normal) */
    uint32_t m = (uint32_t)rint(v / ldexp(1.0, -24));
    return sign | (uint16_t)m;    /* m == 1024 encodes 2^-14 correctly */
  }
  int ev;
  frexp(v, &ev);
  ev -= 1;
  uint32_t frac = (uint32_t)rint((v / ldexp(1.0, ev) - 1.0) * 1024.0);
  return sign | (uint16_t)(((ev + 15) << 10) | frac);
}

/* Symmetric absmax quantiser: scale = fp16(absmax / qmax) (ties to even),
 * code = clamp(round_half_even(x / scale), -qmax, qmax); a zero scale gives
 * zero codes. Writes the scale's fp16 bits. */
static void quantize_block(const double* x, int n, int qmax, int* codes, uint16_t* scale_bits) {
  double amax = 0;
  for (int i = 0; i < n; i++) amax = fmax(amax, fabs(x[i]));
  uint16_t sb = oracle_double_to_f16(amax / (double)qmax);
  double s = oracle_f16_to_double(sb);
  *scale_bits = sb;
  for (int i = 0; i < n; i++) {
    if (s == 0 || isinf(s)) { codes[i] = 0; continue; }
    double c = rint(x[i] / s);
    if (c > qmax) c = qmax;
    if (c < -qmax) c = -qmax;
    codes[i] = (int)c;
  }
}

/* ------------------------------------------------------------------ */
/* Symmetric eigendecomposition: cyclic Jacobi (Golub & Van Loan,       */
/* "Matrix Computations", section 8.5, cyclic-by-row Jacobi).           */
/* ------------------------------------------------------------------ */

/* a: n*n symmetric (destroyed); w: eigenvalues; u: n*n, column k is the
 * eigenvector of w[k]. Returns the number of sweeps used. */
int oracle_jacobi_eigh(int n, double* a, double* w, double* u) {
  for (int i = 0; i < n; i++)
    for (int j = 0; j < n; j++) u[i * n + j] = (i == j) ? 1.0 : 0.0;
  int sweep;
  for (sweep = 0; sweep < 100; sweep++) {
    double off = 0, tot = 0;
    for (int i = 0; i < n; i++)
      for (int j = 0; j < n; j++) {
        double v = a[i * n + j] * a[i * n + j];
        tot += v;
        if (i != j) off += v;
      }
    if (off == 0 || sqrt(off) <= 1e-15 * sqrt(tot)) break;
    for (int p = 0; p < n - 1; p++)
      for (int q = p + 1; q < n; q++) {
        double apq = a[p * n + q];
        if (apq == 0) continue;
        /* symmetric Schur 2x2: choose the rotation that zeroes a[p][q] */
        double tau = (a[q * n + q] - a[p * n + p]) / (2.0 * apq);
        double t = (tau >= 0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
        double c = 1.0 / sqrt(1.0 + t * t), s = t * c;
        /* A <- J^T A J, J = identity except J[p][p]=J[q][q]=c, J[p][q]=s, J[q][p]=-s */
        for (int k = 0; k < n; k++) {
          double akp = a[k * n + p], akq = a[k * n + q];
          a[k * n + p] = c * akp - s * akq;
          a[k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; k++) {
          double apk = a[p * n + k], aqk = a[q * n + k];
          a[p * n + k] = c * apk - s * aqk;
          a[q * n + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < n; k++) {
          double ukp = u[k * n + p], ukq = u[k * n + q];
          u[k * n + p] = c * ukp - s * ukq;
          u[k * n + q] = s * ukp + c * ukq;
        }
      }
  }
  for (int i = 0; i < n; i++) w[i] = a[i * n + i];
  return sweep;
}

/* ------------------------------------------------------------------ */
/* Summary build (A "How LOCKS works" + A "Code" build loop;            */
/* B mechanism 1)                                                       */
/* ------------------------------------------------------------------ */

/* Unquantised rank-r summary of one 16x128 key tile.
 * keys: 16*128 doubles. Outputs mu[128], V[128*r] (column k = basis vector k),
 * C[16*r] (row i = coefficients of token i), lam[16] eigenvalues of the
 * centred Gram, descending. r in 1..16 (the centred keys have rank <= 15, so
 * a 16th direction has zero energy and a zero column). */
void oracle_page_summary_f64(const double* keys, int r, double* mu, double* V, double* C,
                             double* lam) {
  double D[OP * OD], G[OP * OP], w[OP], U[OP * OP];
  /* centroid: mean key over the page's 16 tokens */
  for (int d = 0; d < OD; d++) {
    double s = 0;
    for (int i = 0; i < OP; i++) s += keys[i * OD + d];
    mu[d] = s / OP;
  }
  /* centred deviations */
  for (int i = 0; i < OP; i++)
    for (int d = 0; d < OD; d++) D[i * OD + d] = keys[i * OD + d] - mu[d];
  /* the page's small Gram matrix D D^T (16x16) */
  for (int i = 0; i < OP; i++)
    for (int j = 0; j < OP; j++) {
      double s = 0;
      for (int d = 0; d < OD; d++) s += D[i * OD + d] * D[j * OD + d];
      G[i * OP + j] = s;
    }
  oracle_jacobi_eigh(OP, G, w, U);
  /* order eigenpairs by eigenvalue, descending; equal values keep index order */
  int ord[OP];
  for (int i = 0; i < OP; i++) ord[i] = i;
  for (int i = 1; i < OP; i++) { /* insertion sort: stable */
    int x = ord[i], j = i - 1;
    while (j >= 0 && w[ord[j]] < w[x]) { ord[j + 1] = ord[j]; j--; }
    ord[j + 1] = x;
  }
  for (int k = 0; k < OP; k++) lam[k] = w[ord[k]];
  /* basis: right singular vectors of D, V[:,k] = D^T u_k / sqrt(lambda_k);
   * directions with (numerically) zero energy give a zero column: energy at
   * most 1e-12 of the leading direction's, or at most 1e-24 of the keys' own
   * energy (the level of double rounding in the centring) */
  double energy = 0;
  for (int i = 0; i < OP * OD; i++) energy += keys[i] * keys[i];
  for (int k = 0; k < r; k++) {
    double l = lam[k];
    int keep = (lam[0] > 0) && (l > 1e-12 * lam[0]) && (l > 1e-24 * energy);
    for (int d = 0; d < OD; d++) {
      double s = 0;
      if (keep)
        for (int i = 0; i < OP; i++) s += D[i * OD + d] * U[i * OP + ord[k]];
      V[d * r + k] = keep ? s / sqrt(l) : 0.0;
    }
  }
  /* sign convention: the largest-magnitude entry of each basis vector is
   * positive (lowest d on ties) */
  for (int k = 0; k < r; k++) {
    int dm = 0;
    for (int d = 1; d < OD; d++)
      if (fabs(V[d * r + k]) > fabs(V[dm * r + k])) dm = d;
    if (V[dm * r + k] < 0)
      for (int d = 0; d < OD; d++) V[d * r + k] = -V[d * r + k];
  }
  /* coefficients: the deviations projected on the basis, C = D V */
  for (int i = 0; i < OP; i++)
    for (int k = 0; k < r; k++) {
      double s = 0;
      for (int d = 0; d < OD; d++) s += D[i * OD + d] * V[d * r + k];
      C[i * r + k] = s;
    }
}

/* Pack codes into the 784-byte record (format documented in the C ABI). */
static void pack_record(const int* mu_c, const int* v_c /* [128][8] */, const int* c_c /* [16][8] */,
                        const uint16_t* scales /* 3 */, uint8_t* rec) {
  memset(rec, 0, OSTRIDE);
  for (int k = 0; k < OR; k++)
    for (int w = 0; w < 16; w++)
      for (int b = 0; b < 4; b++) {
        int lo = v_c[(8 * w + b) * OR + k] & 0xf;
        int hi = v_c[(8 * w + 4 + b) * OR + k] & 0xf;
        rec[OV_OFF + k * 64 + w * 4 + b] = (uint8_t)(lo | (hi << 4));
      }
  for (int d = 0; d < OD; d++) rec[OMU_OFF + d] = (uint8_t)(int8_t)mu_c[d];
  for (int i = 0; i < OP * OR; i++) rec[OC_OFF + i] = (uint8_t)(int8_t)c_c[i];
  for (int s = 0; s < 3; s++) {
    rec[OS_OFF + 2 * s] = (uint8_t)(scales[s] & 0xff);
    rec[OS_OFF + 2 * s + 1] = (uint8_t)(scales[s] >> 8);
  }
}

/* Quantised record of one page from its bf16 key tile (16*128 bf16 bits).
 * Optional diagnostics: lam[16] eigenvalues; mu/V/C unquantised (may be NULL). */
void oracle_build_record(const uint16_t* keys_bf16, uint8_t* rec, double* lam_out,
                         double* mu_out, double* v_out, double* c_out) {
  double keys[OP * OD], mu[OD], V[OD * OR], C[OP * OR], lam[OP];
  for (int i = 0; i < OP * OD; i++) keys[i] = oracle_bf16_to_double(keys_bf16[i]);
  oracle_page_summary_f64(keys, OR, mu, V, C, lam);
  int mu_c[OD], v_c[OD * OR], c_c[OP * OR];
  uint16_t sc[3];
  quantize_block(mu, OD, 127, mu_c, &sc[0]);
  quantize_block(V, OD * OR, 7, v_c, &sc[1]);
  quantize_block(C, OP * OR, 127, c_c, &sc[2]);
  pack_record(mu_c, v_c, c_c, sc, rec);
  if (lam_out) memcpy(lam_out, lam, sizeof lam);
  if (mu_out) memcpy(mu_out, mu, sizeof mu);
  if (v_out) memcpy(v_out, V, sizeof V);
  if (c_out) memcpy(c_out, C, sizeof C);
}

/* Decode a record back to doubles: mu[128], V[128*8], C[16*8]. */
void oracle_unpack_record(const uint8_t* rec, double* mu, double* V, double* C) {
  double s_mu = oracle_f16_to_double((uint16_t)(rec[OS_OFF] | (rec[OS_OFF + 1] << 8)));
  double s_v = oracle_f16_to_double((uint16_t)(rec[OS_OFF + 2] | (rec[OS_OFF + 3] << 8)));
  double s_c = oracle_f16_to_double((uint16_t)(rec[OS_OFF + 4] | (rec[OS_OFF + 5] << 8)));
  for (int k = 0; k < OR; k++)
    for (int w = 0; w < 16; w++)
      for (int b = 0; b < 4; b++) {
        uint8_t byte = rec[OV_OFF + k * 64 + w * 4 + b];
        int lo = byte & 0xf, hi = byte >> 4;
        if (lo >= 8) lo -= 16; /* 4-bit two's complement */
        if (hi >= 8) hi -= 16;
        V[(8 * w + b) * OR + k] = s_v * lo;
        V[(8 * w + 4 + b) * OR + k] = s_v * hi;
      }
  for (int d = 0; d < OD; d++) mu[d] = s_mu * (int8_t)rec[OMU_OFF + d];
  for (int i = 0; i < OP * OR; i++) C[i] = s_c * (int8_t)rec[OC_OFF + i];
}

/* ------------------------------------------------------------------ */
/* Variant record formats: the precision / rank ablation (A "Caveats": */
/* Theorem 1 holds for unquantised summaries; int4 loses a few recall   */
/* points, int2 collapses)                                              */
/* ------------------------------------------------------------------ */

/* Rank r in {4, 8, 16}; V in vbits in {2, 4} (signed integer codes, range
 * +-(2^(vbits-1) - 1)) or 16 (fp16 values). mu and C are int8 codes (range
 * +-127) in the integer formats and fp16 values in the fp16 format. Bytes:
 * V [d][k] row-major, element e = d*r + k in bits [e*vbits, (e+1)*vbits)
 * (little-endian; two's complement for codes); then mu[128]; then C[16][r];
 * then fp16 scales {s_mu, s_V, s_C, 0} (1.0 where values are stored as
 * fp16); zero padding to a multiple of 16 bytes. */
static int variant_mbits(int vbits) { return vbits == 16 ? 16 : 8; }

size_t oracle_variant_record_bytes(int r, int vbits) {
  size_t b = (size_t)OD * r * vbits / 8 + (size_t)OD * variant_mbits(vbits) / 8 +
             (size_t)OP * r * variant_mbits(vbits) / 8 + 8;
  return (b + 15) / 16 * 16;
}

static void put_bits(uint8_t* base, size_t e, int bits, uint32_t v) {
  for (int t = 0; t < bits; t++) {
    size_t bit = e * bits + t;
    if ((v >> t) & 1u) base[bit / 8] |= (uint8_t)(1u << (bit % 8));
  }
}

static uint32_t get_bits(const uint8_t* base, size_t e, int bits) {
  uint32_t v = 0;
  for (int t = 0; t < bits; t++) {
    size_t bit = e * bits + t;
    v |= (uint32_t)((base[bit / 8] >> (bit % 8)) & 1u) << t;
  }
  return v;
}

/* One tensor stored as codes (bits < 16, with its quantiser scale) or fp16
 * values (bits = 16, scale 1.0). Returns the scale's fp16 bits. */
static uint16_t store_tensor(const double* x, int n, int bits, uint8_t* dst) {
  if (bits == 16) {
    for (int i = 0; i < n; i++) put_bits(dst, i, 16, oracle_double_to_f16(x[i]));
    return 0x3C00; /* 1.0 */
  }
  int* codes = (int*)malloc(sizeof(int) * n);
  uint16_t sb;
  quantize_block(x, n, (1 << (bits - 1)) - 1, codes, &sb);
  for (int i = 0; i < n; i++) put_bits(dst, i, bits, (uint32_t)codes[i] & ((1u << bits) - 1));
  free(codes);
  return sb;
}

static void load_tensor(const uint8_t* src, int n, int bits, double scale, double* x) {
  for (int i = 0; i < n; i++) {
    uint32_t v = get_bits(src, i, bits);
    if (bits == 16) {
      x[i] = oracle_f16_to_double((uint16_t)v);
    } else {
      int c = (int)v;
      if (c >= (1 << (bits - 1))) c -= 1 << bits; /* two's complement */
      x[i] = scale * c;
    }
  }
}

void oracle_build_record_variant(const uint16_t* keys_bf16, int r, int vbits, uint8_t* rec) {
  double keys[OP * OD], mu[OD], V[OD * 16], C[OP * 16], lam[OP];
  for (int i = 0; i < OP * OD; i++) keys[i] = oracle_bf16_to_double(keys_bf16[i]);
  oracle_page_summary_f64(keys, r, mu, V, C, lam);
  int mb = variant_mbits(vbits);
  size_t ov = 0, om = (size_t)OD * r * vbits / 8, oc = om + (size_t)OD * mb / 8,
         os = oc + (size_t)OP * r * mb / 8;
  memset(rec, 0, oracle_variant_record_bytes(r, vbits));
  uint16_t sc[3];
  sc[1] = store_tensor(V, OD * r, vbits, rec + ov);
  sc[0] = store_tensor(mu, OD, mb, rec + om);
  sc[2] = store_tensor(C, OP * r, mb, rec + oc);
  for (int t = 0; t < 3; t++) {
    rec[os + 2 * t] = (uint8_t)(sc[t] & 0xff);
    rec[os + 2 * t + 1] = (uint8_t)(sc[t] >> 8);
  }
}

/* Decode a variant record: mu[128], V[128*r], C[16*r]. */
void oracle_unpack_record_variant(const uint8_t* rec, int r, int vbits, double* mu, double* V,
                                  double* C) {
  int mb = variant_mbits(vbits);
  size_t om = (size_t)OD * r * vbits / 8, oc = om + (size_t)OD * mb / 8,
         os = oc + (size_t)OP * r * mb / 8;
  double s_mu = oracle_f16_to_double((uint16_t)(rec[os] | (rec[os + 1] << 8)));
  double s_v = oracle_f16_to_double((uint16_t)(rec[os + 2] | (rec[os + 3] << 8)));
  double s_c = oracle_f16_to_double((uint16_t)(rec[os + 4] | (rec[os + 5] << 8)));
  load_tensor(rec, OD * r, vbits, s_v, V);
  load_tensor(rec + om, OD, mb, s_mu, mu);
  load_tensor(rec + oc, OP * r, mb, s_c, C);
}

/* Variant records of every full page of every sequence (stride = the
 * variant's record bytes); records of unreferenced blocks are untouched. */
void oracle_build_summaries_variant(int B, int Hkv, int max_pages, int num_blocks,
                                    const uint16_t* k_cache, const int32_t* page_table,
                                    const int32_t* seq_lens, int r, int vbits,
                                    uint8_t* summaries) {
  size_t stride = oracle_variant_record_bytes(r, vbits);
  for (int b = 0; b < B; b++) {
    int n = seq_lens[b] / OP;
    if (n > max_pages) n = max_pages;
    if (n < 0) n = 0;
#pragma omp parallel for schedule(dynamic, 64)
    for (int u = 0; u < n * Hkv; u++) {
      int j = u / Hkv, kvh = u % Hkv;
      int blk = page_table[(size_t)b * max_pages + j];
      if (blk < 0 || blk >= num_blocks) continue;
      const uint16_t* tile = k_cache + ((size_t)blk * Hkv + kvh) * OP * OD;
      oracle_build_record_variant(tile, r, vbits, summaries + ((size_t)blk * Hkv + kvh) * stride);
    }
  }
}

/* ------------------------------------------------------------------ */
/* The shared-basis comparison of Proposition 1 (A "Why shared-basis    */
/* sparse attention is structurally broken"; B section 3 theory): a     */
/* selector that scores pages through one fixed projection W shared by */
/* all pages of a sequence, in the same page-score form as LOCKS.       */
/* ------------------------------------------------------------------ */

/* Record of one page under a fixed shared basis W (128 x r, row-major
 * [d][k]): centroid mu = mean of the 16 keys, coefficients C = (K - 1 mu^T) W
 * (the deviations projected onto W), V = W. Stored in the variant layout with
 * fp16 values (v_bits 16, scales 1.0), so the variant score reads it. */
void oracle_build_record_shared(const uint16_t* keys_bf16, const double* W, int r, uint8_t* rec) {
  double keys[OP * OD], mu[OD], C[OP * 16];
  for (int i = 0; i < OP * OD; i++) keys[i] = oracle_bf16_to_double(keys_bf16[i]);
  for (int d = 0; d < OD; d++) {
    double m = 0;
    for (int i = 0; i < OP; i++) m += keys[i * OD + d];
    mu[d] = m / OP;
  }
  for (int i = 0; i < OP; i++)
    for (int k = 0; k < r; k++) {
      double c = 0;
      for (int d = 0; d < OD; d++) c += (keys[i * OD + d] - mu[d]) * W[d * r + k];
      C[i * r + k] = c;
    }
  size_t om = (size_t)OD * r * 2, oc = om + (size_t)OD * 2, os = oc + (size_t)OP * r * 2;
  memset(rec, 0, oracle_variant_record_bytes(r, 16));
  store_tensor(W, OD * r, 16, rec);
  store_tensor(mu, OD, 16, rec + om);
  store_tensor(C, OP * r, 16, rec + oc);
  for (int t = 0; t < 3; t++) {
    rec[os + 2 * t] = 0x00;
    rec[os + 2 * t + 1] = 0x3C; /* fp16 1.0 */
  }
}

/* Shared-basis records of every full page: the page's sequence b and KV head
 * select its basis, basis[b][kvh] (128 x r, row-major). */
void oracle_build_summaries_shared(int B, int Hkv, int max_pages, int num_blocks,
                                   const uint16_t* k_cache, const int32_t* page_table,
                                   const int32_t* seq_lens, const double* basis, int r,
                                   uint8_t* summaries) {
  size_t stride = oracle_variant_record_bytes(r, 16);
  for (int b = 0; b < B; b++) {
    int n = seq_lens[b] / OP;
    if (n > max_pages) n = max_pages;
    if (n < 0) n = 0;
#pragma omp parallel for schedule(dynamic, 64)
    for (int u = 0; u < n * Hkv; u++) {
      int j = u / Hkv, kvh = u % Hkv;
      int blk = page_table[(size_t)b * max_pages + j];
      if (blk < 0 || blk >= num_blocks) continue;
      const uint16_t* tile = k_cache + ((size_t)blk * Hkv + kvh) * OP * OD;
      oracle_build_record_shared(tile, basis + ((size_t)b * Hkv + kvh) * OD * r, r,
                                 summaries + ((size_t)blk * Hkv + kvh) * stride);
    }
  }
}

/* The basis a sequence-level shared projection would use: for each
 * (sequence, KV head), the top-r eigenvectors (eigenvalues descending, ties
 * by index) of the pooled within-page deviation scatter sum_j D_j^T D_j over
 * the sequence's full, present pages, D_j = K_j - 1 mu_j^T. Written as
 * basis[b][kvh] (128 x r, row-major [d][k]), each column's largest-|.|
 * entry made positive (lowest d on ties). */
void oracle_shared_basis(int B, int Hkv, int max_pages, int num_blocks, const uint16_t* k_cache,
                         const int32_t* page_table, const int32_t* seq_lens, int r,
                         double* basis) {
  double* S = (double*)malloc(sizeof(double) * OD * OD);
  double* U = (double*)malloc(sizeof(double) * OD * OD);
  double w[OD];
  for (int b = 0; b < B; b++) {
    int n = seq_lens[b] / OP;
    if (n > max_pages) n = max_pages;
    if (n < 0) n = 0;
    for (int kvh = 0; kvh < Hkv; kvh++) {
      memset(S, 0, sizeof(double) * OD * OD);
      for (int j = 0; j < n; j++) {
        int blk = page_table[(size_t)b * max_pages + j];
        if (blk < 0 || blk >= num_blocks) continue;
        const uint16_t* tile = k_cache + ((size_t)blk * Hkv + kvh) * OP * OD;
        double keys[OP * OD], mu[OD];
        for (int i = 0; i < OP * OD; i++) keys[i] = oracle_bf16_to_double(tile[i]);
        for (int d = 0; d < OD; d++) {
          double m = 0;
          for (int i = 0; i < OP; i++) m += keys[i * OD + d];
          mu[d] = m / OP;
        }
        for (int i = 0; i < OP; i++)
          for (int d = 0; d < OD; d++) keys[i * OD + d] -= mu[d];
        for (int x = 0; x < OD; x++)
          for (int y = 0; y < OD; y++) {
            double acc = 0;
            for (int i = 0; i < OP; i++) acc += keys[i * OD + x] * keys[i * OD + y];
            S[x * OD + y] += acc;
          }
      }
      oracle_jacobi_eigh(OD, S, w, U);
      int order[OD];
      for (int i = 0; i < OD; i++) order[i] = i;
      for (int i = 1; i < OD; i++) { /* stable insertion sort, descending */
        int v = order[i], j = i - 1;
        while (j >= 0 && w[order[j]] < w[v]) {
          order[j + 1] = order[j];
          j--;
        }
        order[j + 1] = v;
      }
      double* dst = basis + ((size_t)b * Hkv + kvh) * OD * r;
      for (int k = 0; k < r; k++) {
        int c = order[k], arg = 0;
        for (int d = 1; d < OD; d++)
          if (fabs(U[d * OD + c]) > fabs(U[arg * OD + c])) arg = d;
        double sg = U[arg * OD + c] < 0 ? -1.0 : 1.0;
        for (int d = 0; d < OD; d++) dst[d * r + k] = sg * U[d * OD + c];
      }
    }
  }
  free(S);
  free(U);
}

/* Summaries of every full page of every sequence; records of unreferenced
 * blocks are left untouched. */
void oracle_build_summaries(int B, int Hkv, int max_pages, int num_blocks,
                            const uint16_t* k_cache, const int32_t* page_table,
                            const int32_t* seq_lens, uint8_t* summaries) {
  for (int b = 0; b < B; b++) {
    int n = seq_lens[b] / OP;
    if (n > max_pages) n = max_pages;
    if (n < 0) n = 0;
#pragma omp parallel for schedule(dynamic, 64)
    for (int u = 0; u < n * Hkv; u++) {
      int j = u / Hkv, kvh = u % Hkv;
      int blk = page_table[(size_t)b * max_pages + j];
      if (blk < 0 || blk >= num_blocks) continue;
      const uint16_t* tile = k_cache + ((size_t)blk * Hkv + kvh) * OP * OD;
      oracle_build_record(tile, summaries + ((size_t)blk * Hkv + kvh) * OSTRIDE, 0, 0, 0, 0);
    }
  }
}

/* ------------------------------------------------------------------ */
/* Page score (A "How LOCKS works" page-score equation; A "Code"        */
/* scoring loop; B mechanism 2)                                         */
/* ------------------------------------------------------------------ */

/* s_hat(q) = log sum_{i in page} exp((q.mu + (V^T q).c_i) / sqrt(d)).
 * V is [128][r] (column k = basis vector k), C is [16][r]. */
double oracle_page_score_f64(const double* q, const double* mu, const double* V,
                             const double* C, int r) {
  const double scale = 1.0 / sqrt((double)OD);
  double global_t = 0;
  for (int d = 0; d < OD; d++) global_t += q[d] * mu[d];
  global_t *= scale;
  double p[16];
  for (int k = 0; k < r; k++) {
    double s = 0;
    for (int d = 0; d < OD; d++) s += V[d * r + k] * q[d];
    p[k] = s;
  }
  double t[OP], m = -INFINITY;
  for (int i = 0; i < OP; i++) {
    double local = 0;
    for (int k = 0; k < r; k++) local += C[i * r + k] * p[k];
    t[i] = global_t + local * scale;
    if (t[i] > m) m = t[i];
  }
  double s = 0;
  for (int i = 0; i < OP; i++) s += exp(t[i] - m);
  return m + log(s);
}

/* The exact per-page log-sum-exp of q.k/sqrt(d) over the page's real keys
 * (the selector that reads every key, B section 3 experiments). */
double oracle_exact_page_lse(const double* q, const double* keys) {
  const double scale = 1.0 / sqrt((double)OD);
  double t[OP], m = -INFINITY;
  for (int i = 0; i < OP; i++) {
    double s = 0;
    for (int d = 0; d < OD; d++) s += q[d] * keys[i * OD + d];
    t[i] = s * scale;
    if (t[i] > m) m = t[i];
  }
  double s = 0;
  for (int i = 0; i < OP; i++) s += exp(t[i] - m);
  return m + log(s);
}

static int valid_pages(const int32_t* seq_lens, int b, int max_pages) {
  int n = seq_lens[b] / OP;
  if (n > max_pages) n = max_pages;
  return n < 0 ? 0 : n;
}

/* Scores of every (sequence, query head, page) from packed summaries.
 * scores: [B][Hq][max_pages]; pages j >= n_b and absent pages get -inf. */
void oracle_scores(int B, int Hq, int Hkv, int max_pages, int num_blocks, const float* q,
                   const uint8_t* summaries, const int32_t* page_table, const int32_t* seq_lens,
                   double* scores) {
  int G = Hq / Hkv;
  for (int b = 0; b < B; b++) {
    int n = valid_pages(seq_lens, b, max_pages);
#pragma omp parallel for schedule(dynamic, 64)
    for (int u = 0; u < max_pages * Hkv; u++) {
      int j = u / Hkv, kvh = u % Hkv;
      int blk = (j < n) ? page_table[(size_t)b * max_pages + j] : -1;
      double mu[OD], V[OD * OR], C[OP * OR];
      int present = blk >= 0 && blk < num_blocks;
      if (present) oracle_unpack_record(summaries + ((size_t)blk * Hkv + kvh) * OSTRIDE, mu, V, C);
      for (int g = 0; g < G; g++) {
        int h = kvh * G + g;
        double qd[OD];
        for (int d = 0; d < OD; d++) qd[d] = q[((size_t)b * Hq + h) * OD + d];
        scores[((size_t)b * Hq + h) * max_pages + j] =
            present ? oracle_page_score_f64(qd, mu, V, C, OR) : -INFINITY;
      }
    }
  }
}

/* Exact page scores: the log-sum-exp of q.k/sqrt(d) over every full page's
 * real keys (the exact-mass selector that Theorem 1 compares LOCKS against,
 * A "How LOCKS works"; B section 3). scores: [B][Hq][max_pages]; pages
 * j >= n_b and absent pages get -inf. */
void oracle_exact_scores(int B, int Hq, int Hkv, int max_pages, int num_blocks, const float* q,
                         const uint16_t* k_cache, const int32_t* page_table,
                         const int32_t* seq_lens, double* scores) {
  int G = Hq / Hkv;
  for (int b = 0; b < B; b++) {
    int n = valid_pages(seq_lens, b, max_pages);
#pragma omp parallel for schedule(dynamic, 64)
    for (int u = 0; u < max_pages * Hkv; u++) {
      int j = u / Hkv, kvh = u % Hkv;
      int blk = (j < n) ? page_table[(size_t)b * max_pages + j] : -1;
      int present = blk >= 0 && blk < num_blocks;
      double keys[OP * OD];
      if (present) {
        const uint16_t* kt = k_cache + ((size_t)blk * Hkv + kvh) * OP * OD;
        for (int x = 0; x < OP * OD; x++) keys[x] = oracle_bf16_to_double(kt[x]);
      }
      for (int g = 0; g < G; g++) {
        int h = kvh * G + g;
        double qd[OD];
        for (int d = 0; d < OD; d++) qd[d] = q[((size_t)b * Hq + h) * OD + d];
        scores[((size_t)b * Hq + h) * max_pages + j] =
            present ? oracle_exact_page_lse(qd, keys) : -INFINITY;
      }
    }
  }
}

/* Page scores from variant records (the page-score equation at rank r). */
void oracle_scores_variant(int B, int Hq, int Hkv, int max_pages, int num_blocks, const float* q,
                           const uint8_t* summaries, int r, int vbits,
                           const int32_t* page_table, const int32_t* seq_lens, double* scores) {
  int G = Hq / Hkv;
  size_t stride = oracle_variant_record_bytes(r, vbits);
  for (int b = 0; b < B; b++) {
    int n = valid_pages(seq_lens, b, max_pages);
#pragma omp parallel for schedule(dynamic, 64)
    for (int u = 0; u < max_pages * Hkv; u++) {
      int j = u / Hkv, kvh = u % Hkv;
      int blk = (j < n) ? page_table[(size_t)b * max_pages + j] : -1;
      double mu[OD], V[OD * 16], C[OP * 16];
      int present = blk >= 0 && blk < num_blocks;
      if (present)
        oracle_unpack_record_variant(summaries + ((size_t)blk * Hkv + kvh) * stride, r, vbits, mu, V, C);
      for (int g = 0; g < G; g++) {
        int h = kvh * G + g;
        double qd[OD];
        for (int d = 0; d < OD; d++) qd[d] = q[((size_t)b * Hq + h) * OD + d];
        scores[((size_t)b * Hq + h) * max_pages + j] =
            present ? oracle_page_score_f64(qd, mu, V, C, r) : -INFINITY;
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* Group-shared selection (B mechanism 3) and top-k (A "Code")          */
/* ------------------------------------------------------------------ */

/* key[b][kvh][j] = log( (1/G) sum_g exp(s_hat[g][j] - L_g) ), with
 * L_g = log sum_j exp(s_hat[g][j]) over the sequence's pages: the log of the
 * group-mean normalised mass share. Absent pages keep -inf. */
void oracle_group_keys(int B, int Hq, int Hkv, int max_pages, const double* scores,
                       double* keys) {
  int G = Hq / Hkv;
  for (int b = 0; b < B; b++)
    for (int kvh = 0; kvh < Hkv; kvh++) {
      double L[64];
      for (int g = 0; g < G; g++) {
        const double* s = scores + ((size_t)b * Hq + kvh * G + g) * max_pages;
        double m = -INFINITY;
        for (int j = 0; j < max_pages; j++) m = fmax(m, s[j]);
        double acc = 0;
        if (m > -INFINITY)
          for (int j = 0; j < max_pages; j++) acc += exp(s[j] - m);
        L[g] = (m > -INFINITY) ? m + log(acc) : -INFINITY;
      }
      for (int j = 0; j < max_pages; j++) {
        double e[64], m = -INFINITY;
        for (int g = 0; g < G; g++) {
          double sj = scores[((size_t)b * Hq + kvh * G + g) * max_pages + j];
          e[g] = (sj > -INFINITY) ? sj - L[g] : -INFINITY;
          m = fmax(m, e[g]);
        }
        double acc = 0;
        if (m > -INFINITY)
          for (int g = 0; g < G; g++) acc += exp(e[g] - m);
        keys[((size_t)b * Hkv + kvh) * max_pages + j] =
            (m > -INFINITY) ? m + log(acc) - log((double)G) : -INFINITY;
      }
    }
}

typedef struct { double key; int id; } keyed;
static int cmp_keyed(const void* x, const void* y) {
  const keyed* a = (const keyed*)x;
  const keyed* b = (const keyed*)y;
  if (a->key > b->key) return -1; /* larger key first */
  if (a->key < b->key) return 1;
  return (a->id > b->id) - (a->id < b->id); /* then lower page id */
}
static int cmp_int(const void* x, const void* y) {
  int a = *(const int*)x, b = *(const int*)y;
  return (a > b) - (a < b);
}

/* selected[b][kvh][0..k): the k largest keys (ties to the lower id), sorted
 * ascending; -inf keys are never selected; unused slots are -1. */
void oracle_select(int B, int Hkv, int max_pages, const double* keys, int k, int32_t* selected) {
  keyed* buf = (keyed*)malloc(sizeof(keyed) * (size_t)(max_pages > 0 ? max_pages : 1));
  int* ids = (int*)malloc(sizeof(int) * (size_t)(k > 0 ? k : 1));
  for (int b = 0; b < B; b++)
    for (int kvh = 0; kvh < Hkv; kvh++) {
      const double* kk = keys + ((size_t)b * Hkv + kvh) * max_pages;
      int n = 0;
      for (int j = 0; j < max_pages; j++)
        if (kk[j] > -INFINITY) { buf[n].key = kk[j]; buf[n].id = j; n++; }
      qsort(buf, (size_t)n, sizeof(keyed), cmp_keyed);
      int m = n < k ? n : k;
      for (int i = 0; i < m; i++) ids[i] = buf[i].id;
      qsort(ids, (size_t)m, sizeof(int), cmp_int);
      int32_t* out = selected + ((size_t)b * Hkv + kvh) * k;
      for (int i = 0; i < k; i++) out[i] = (i < m) ? ids[i] : -1;
    }
  free(buf);
  free(ids);
}

/* ------------------------------------------------------------------ */
/* Attention (A "Code": exact attention over the gathered tokens of the */
/* kept pages; with every page kept it is the dense full-KV attention)  */
/* ------------------------------------------------------------------ */

/* Tokens of sequence b past its last full page: they sit in logical page
 * n_b, which has no summary yet (a summary is built when its page fills). */
static int tail_tokens(const int32_t* seq_lens, int b, int max_pages) {
  int n = valid_pages(seq_lens, b, max_pages);
  if (n >= max_pages || seq_lens[b] <= 0) return 0;
  return seq_lens[b] - n * OP;
}

/* out[b][h][128] = softmax_t(q_h . k_t / sqrt(128)) v_t over the tokens of the
 * pages listed in sel[b][kvh][0..k) (entries < 0 or >= n_b skipped) and the
 * tail tokens of the partly filled page n_b. With sel == NULL every full page
 * of the sequence is used (dense attention over all seq_len tokens). Heads
 * with no token get 0. */
void oracle_attention(int B, int Hq, int Hkv, int max_pages, int num_blocks, const float* q,
                      const uint16_t* k_cache, const uint16_t* v_cache,
                      const int32_t* page_table, const int32_t* seq_lens, const int32_t* sel,
                      int k, double* out) {
  int G = Hq / Hkv;
  const double scale = 1.0 / sqrt((double)OD);
  for (int b = 0; b < B; b++) {
    int n = valid_pages(seq_lens, b, max_pages);
    int tail = tail_tokens(seq_lens, b, max_pages);
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < Hq; h++) {
      int kvh = h / G;
      int npg = sel ? k : n;
      /* the attended (block, token count) list: listed pages, then the tail */
      int* blk_of = (int*)malloc(sizeof(int) * (npg + 1));
      int* ntok_of = (int*)malloc(sizeof(int) * (npg + 1));
      int ne = 0;
      for (int s = 0; s < npg; s++) {
        int j = sel ? sel[((size_t)b * Hkv + kvh) * k + s] : s;
        if (j < 0 || j >= n) continue;
        int blk = page_table[(size_t)b * max_pages + j];
        if (blk < 0 || blk >= num_blocks) continue;
        blk_of[ne] = blk;
        ntok_of[ne++] = OP;
      }
      if (tail > 0) {
        int blk = page_table[(size_t)b * max_pages + n];
        if (blk >= 0 && blk < num_blocks) {
          blk_of[ne] = blk;
          ntok_of[ne++] = tail;
        }
      }
      double qd[OD];
      for (int d = 0; d < OD; d++) qd[d] = q[((size_t)b * Hq + h) * OD + d];
      /* pass 1: the maximum logit */
      double m = -INFINITY;
      for (int e = 0; e < ne; e++) {
        const uint16_t* kt = k_cache + ((size_t)blk_of[e] * Hkv + kvh) * OP * OD;
        for (int i = 0; i < ntok_of[e]; i++) {
          double l = 0;
          for (int d = 0; d < OD; d++) l += qd[d] * oracle_bf16_to_double(kt[i * OD + d]);
          m = fmax(m, l * scale);
        }
      }
      double o[OD], den = 0;
      for (int d = 0; d < OD; d++) o[d] = 0;
      if (m > -INFINITY) {
        /* pass 2: softmax weights and the weighted sum of values */
        for (int e = 0; e < ne; e++) {
          const uint16_t* kt = k_cache + ((size_t)blk_of[e] * Hkv + kvh) * OP * OD;
          const uint16_t* vt = v_cache + ((size_t)blk_of[e] * Hkv + kvh) * OP * OD;
          for (int i = 0; i < ntok_of[e]; i++) {
            double l = 0;
            for (int d = 0; d < OD; d++) l += qd[d] * oracle_bf16_to_double(kt[i * OD + d]);
            double w = exp(l * scale - m);
            den += w;
            for (int d = 0; d < OD; d++) o[d] += w * oracle_bf16_to_double(vt[i * OD + d]);
          }
        }
      }
      for (int d = 0; d < OD; d++)
        out[((size_t)b * Hq + h) * OD + d] = (den > 0) ? o[d] / den : 0.0;
      free(blk_of);
      free(ntok_of);
    }
  }
}

/* The whole decode step on packed summaries: scores -> group keys -> top-k ->
 * attention over the kept pages. Any of scores_out / keys_out may be NULL. */
void oracle_decode_step(int B, int Hq, int Hkv, int max_pages, int num_blocks, const float* q,
                        const uint8_t* summaries, const uint16_t* k_cache,
                        const uint16_t* v_cache, const int32_t* page_table,
                        const int32_t* seq_lens, int budget_tokens, double* out,
                        int32_t* selected, double* scores_out, double* keys_out) {
  int k = budget_tokens / OP;
  size_t ns = (size_t)B * Hq * max_pages, nk = (size_t)B * Hkv * max_pages;
  double* scores = scores_out ? scores_out : (double*)malloc(sizeof(double) * (ns ? ns : 1));
  double* keys = keys_out ? keys_out : (double*)malloc(sizeof(double) * (nk ? nk : 1));
  oracle_scores(B, Hq, Hkv, max_pages, num_blocks, q, summaries, page_table, seq_lens, scores);
  oracle_group_keys(B, Hq, Hkv, max_pages, scores, keys);
  oracle_select(B, Hkv, max_pages, keys, k, selected);
  oracle_attention(B, Hq, Hkv, max_pages, num_blocks, q, k_cache, v_cache, page_table, seq_lens,
                   selected, k, out);
  if (!scores_out) free(scores);
  if (!keys_out) free(keys);
}

/* Threads the OpenMP loops above use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
