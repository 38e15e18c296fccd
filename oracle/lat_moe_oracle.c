/*
 * CPU oracle for the quantized latent-MoE expert stage.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may call,
 * link or load this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP implementation.
 *
 * What it computes (the expert stage of a latent layer's prompt path):
 *   for every routed pair p = (token t, slot j) with expert e = idx[t][j]:
 *     gate/up  : Q3_K weights [2F][L] against the token's q8_1 latent row,
 *                as integer dots per 32-value activation block, scales
 *                folded in floating point,
 *     SwiGLU   : H = silu(G) * U,
 *     requant  : H re-rounded to q8_1 (32-value blocks),
 *     down     : IQ4_NL weights [L][F] against H, same block structure
 *                (or Q4_0 weights, the same block layout with a linear
 *                table: see orc_q4_0_decode),
 *     combine  : y[t] += w[t][j] * O, slots taken in order j = 0..k-1.
 * Source: "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section
 * "Contents" (gate/up reads Q3_K, applies SwiGLU and rounds H to q8_1; down
 * reads IQ4_NL) and the lat_q3k_w11.cu commit message (the same pipeline,
 * each expert's weights read in place, and the sub-block scale folded into
 * the integer operand as (4 - code) * (scale - 32), range [-128, 124], so one
 * integer dot covers a whole 32-value activation block).  Grouping tokens by
 * expert is a scheduling choice that does not change the result, so the
 * oracle simply walks the pairs token by token.
 *
 * It also computes the two dense projections around the stage in a latent
 * layer (D: hidden row -> latent row, stored as q8_1; U: latent row ->
 * hidden row), Q8_0 weights against q8_1 activations with the same block
 * structure (see the section near the end of the file).
 *
 * The Q3_K / IQ4_NL / q8_1 / Q8_0 bit layouts are ggml's public GGUF block formats;
 * the pages name them without restating them.  They are restated here from
 * that specification.
 *
 * Precision: every scale fold, the SwiGLU and the down projection run in
 * fp64.  The one place where floating point decides an integer -- the q8_1
 * rounding of H (and of the input activations) -- is taken in fp32 with
 * IEEE operations in a fixed order, the same precision the GPU kernel uses,
 * so both sides make that decision from the same rule:
 *     amax = max |v|;  d = amax / 127;  id = (d != 0) ? 1 / d : 0;
 *     q = round_half_away_from_zero(v * id);  stored d = fp16_rne(d);
 *     stored s = fp16_rne(d * sum(q)).
 * Build with -ffp-contract=off so no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q3K_BYTES 110
#define Q3K_VALUES 256
#define IQ4NL_BYTES 18
#define IQ4NL_VALUES 32
#define Q81_BYTES 36
#define Q81_VALUES 32

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp32/fp64 (IEEE binary16)                                        */
/* ------------------------------------------------------------------------ */

/* Exact value of an IEEE binary16 bit pattern. */
double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (exp == 0) {
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man | 0x400), exp - 25); /* (1024 + man) * 2^(exp-25) */
  }
  return sign ? -v : v;
}

/* fp32 -> binary16, round to nearest, ties to even. */
uint16_t orc_float_to_half(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u));
  uint32_t e = ax >> 23;           /* biased fp32 exponent */
  uint32_t m = ax & 0x7fffffu;
  if (e >= 113) {                  /* |f| >= 2^-14: normal binary16 range (or overflow) */
    uint32_t h = ((e - 112) << 10) | (m >> 13);
    uint32_t rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
    if (h >= 0x7c00u) h = 0x7c00u; /* rounds to infinity */
    return (uint16_t)(sign | h);
  }
  /* subnormal binary16: count units of 2^-24 */
  if (e == 0) return (uint16_t)sign; /* fp32 subnormals are far below 2^-25 */
  uint32_t full = m | 0x800000u;     /* value = full * 2^(e-150) */
  uint32_t shift = 126 - e;          /* units of 2^-24: full >> shift */
  if (shift > 24) return (uint16_t)sign;
  uint32_t q = full >> shift;
  uint32_t rem = full & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;
  return (uint16_t)(sign | q);
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xff);
  p[1] = (uint8_t)(v >> 8);
}

/* ------------------------------------------------------------------------ */
/* Block decoders                                                             */
/* ------------------------------------------------------------------------ */

/* Q3_K: 256 weights in 110 bytes = hmask[32] | qs[64] | scales[12] | d (fp16).
 * Element i = 128*n + 32*j + l (n in 0..1, j in 0..3, l in 0..31):
 *   low two bits  = (qs[32*n + l] >> (2*j)) & 3
 *   high bit      = (hmask[l] >> (4*n + j)) & 1
 *   code c        = low + 4*high in 0..7, signed value v = c - 4 in -4..3
 * Sub-block s = i / 16 has a 6-bit scale:
 *   low nibble = s < 8 ? scales[s] & 15 : scales[s - 8] >> 4
 *   top bits   = (scales[8 + s % 4] >> (2 * (s / 4))) & 3
 *   sigma      = (low | top << 4) - 32 in -32..31
 * Weight i = d * sigma(i / 16) * v(i). */
void orc_q3k_decode(const uint8_t* blk, int8_t* v, int8_t* sigma, double* d) {
  const uint8_t* hmask = blk;
  const uint8_t* qs = blk + 32;
  const uint8_t* sc = blk + 96;
  for (int i = 0; i < Q3K_VALUES; ++i) {
    int n = i / 128, j = (i % 128) / 32, l = i % 32;
    int low = (qs[32 * n + l] >> (2 * j)) & 3;
    int high = (hmask[l] >> (4 * n + j)) & 1;
    v[i] = (int8_t)(low + 4 * high - 4);
  }
  for (int s = 0; s < 16; ++s) {
    int lo = s < 8 ? (sc[s] & 15) : (sc[s - 8] >> 4);
    int hi = (sc[8 + s % 4] >> (2 * (s / 4))) & 3;
    sigma[s] = (int8_t)((lo | (hi << 4)) - 32);
  }
  *d = orc_half_to_double(rd16(blk + 108));
}

/* IQ4_NL: 32 weights in 18 bytes = d (fp16) | qs[16].  Element i < 16 uses
 * the low nibble of qs[i], element i >= 16 the high nibble of qs[i - 16];
 * the nibble indexes a fixed 16-entry non-linear table.  Weight = d * K. */
static const int8_t IQ4NL_TABLE[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                       1,    13,   25,  38,  53,  69,  89,  113};

void orc_iq4nl_decode(const uint8_t* blk, int8_t* kv, double* d) {
  const uint8_t* qs = blk + 2;
  for (int i = 0; i < IQ4NL_VALUES; ++i) {
    int nib = i < 16 ? (qs[i] & 15) : (qs[i - 16] >> 4);
    kv[i] = IQ4NL_TABLE[nib];
  }
  *d = orc_half_to_double(rd16(blk));
}

/* Q4_0: 32 weights in 18 bytes = d (fp16) | qs[16], the nibbles in the same
 * places as IQ4_NL's; weight = d * (nibble - 8).  The format is one of the
 * weight formats the PR page names ("Not done": a Q4_0 file was not tried);
 * its layout is ggml's public GGUF definition.  Here it is an alternative
 * format of the down weights. */
void orc_q4_0_decode(const uint8_t* blk, int8_t* v, double* d) {
  const uint8_t* qs = blk + 2;
  for (int i = 0; i < IQ4NL_VALUES; ++i) {
    int nib = i < 16 ? (qs[i] & 15) : (qs[i - 16] >> 4);
    v[i] = (int8_t)(nib - 8);
  }
  *d = orc_half_to_double(rd16(blk));
}

/* Down weight formats (both 18 bytes per 32 weights). */
#define DOWN_IQ4NL 0
#define DOWN_Q4_0 1
static void down_block_decode(int fmt, const uint8_t* blk, int8_t* kv, double* d) {
  if (fmt == DOWN_Q4_0)
    orc_q4_0_decode(blk, kv, d);
  else
    orc_iq4nl_decode(blk, kv, d);
}

/* q8_1: 32 values in 36 bytes = d (fp16) | s (fp16) | qs[32] (int8). */
void orc_q8_1_decode(const uint8_t* blk, int8_t* q, double* d) {
  for (int i = 0; i < Q81_VALUES; ++i) q[i] = (int8_t)blk[4 + i];
  *d = orc_half_to_double(rd16(blk));
}

/* Round to q8_1 in fp32 (the rule in the file header). */
void orc_q8_1_quantize_block(const float* x, uint8_t* out) {
  float amax = 0.0f;
  for (int i = 0; i < Q81_VALUES; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 127.0f;
  float id = d != 0.0f ? 1.0f / d : 0.0f;
  int sum = 0;
  for (int i = 0; i < Q81_VALUES; ++i) {
    float prod = x[i] * id;
    int q = (int)roundf(prod); /* C roundf: halfway cases away from zero */
    out[4 + i] = (uint8_t)(int8_t)q;
    sum += q;
  }
  wr16(out, orc_float_to_half(d));
  wr16(out + 2, orc_float_to_half(d * (float)sum));
}

/* x [rows][cols] fp32 -> q8_1 blocks [rows][cols/32]. */
void orc_quantize_q8_1(const float* x, int64_t rows, int32_t cols, uint8_t* out) {
  int64_t nb = (int64_t)cols / Q81_VALUES;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      orc_q8_1_quantize_block(x + r * cols + b * Q81_VALUES, out + (r * nb + b) * Q81_BYTES);
}

/* Dequantized values (exact in fp64): used by the brute-force dense checks. */
void orc_dequant_q3k(const uint8_t* blocks, int64_t nblocks, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblocks; ++b) {
    int8_t v[Q3K_VALUES], sg[16];
    double d;
    orc_q3k_decode(blocks + b * Q3K_BYTES, v, sg, &d);
    for (int i = 0; i < Q3K_VALUES; ++i) out[b * Q3K_VALUES + i] = d * (double)sg[i / 16] * (double)v[i];
  }
}
void orc_dequant_iq4nl(const uint8_t* blocks, int64_t nblocks, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblocks; ++b) {
    int8_t kv[IQ4NL_VALUES];
    double d;
    orc_iq4nl_decode(blocks + b * IQ4NL_BYTES, kv, &d);
    for (int i = 0; i < IQ4NL_VALUES; ++i) out[b * IQ4NL_VALUES + i] = d * (double)kv[i];
  }
}
void orc_dequant_q4_0(const uint8_t* blocks, int64_t nblocks, double* out) {
  for (int64_t b = 0; b < nblocks; ++b) {
    double d;
    int8_t v[IQ4NL_VALUES];
    orc_q4_0_decode(blocks + b * IQ4NL_BYTES, v, &d);
    for (int i = 0; i < IQ4NL_VALUES; ++i) out[b * IQ4NL_VALUES + i] = d * (double)v[i];
  }
}

void orc_dequant_q8_1(const uint8_t* blocks, int64_t nblocks, double* out) {
  for (int64_t b = 0; b < nblocks; ++b) {
    int8_t q[Q81_VALUES];
    double d;
    orc_q8_1_decode(blocks + b * Q81_BYTES, q, &d);
    for (int i = 0; i < Q81_VALUES; ++i) out[b * Q81_VALUES + i] = d * (double)q[i];
  }
}
/* Decoded fields, for format tests: v/sigma per block, table values. */
void orc_q3k_fields(const uint8_t* blocks, int64_t nblocks, int8_t* v, int8_t* sigma, double* d) {
  for (int64_t b = 0; b < nblocks; ++b)
    orc_q3k_decode(blocks + b * Q3K_BYTES, v + b * Q3K_VALUES, sigma + b * 16, d + b);
}
void orc_iq4nl_fields(const uint8_t* blocks, int64_t nblocks, int8_t* kv, double* d) {
  for (int64_t b = 0; b < nblocks; ++b) orc_iq4nl_decode(blocks + b * IQ4NL_BYTES, kv + b * IQ4NL_VALUES, d + b);
}

/* ------------------------------------------------------------------------ */
/* Integer block dots                                                         */
/* ------------------------------------------------------------------------ */

/* Gate/up block dots of one weight row against one q8_1 activation row:
 *   I32[b] = sum over the 32 values i of block b of sigma(i/16) * v(i) * q(i)
 *   I16[s] = sum over the 16 values i of sub-block s of v(i) * q(i)
 * Row = L/256 Q3_K blocks; act = L/32 q8_1 blocks.  dw[sb] gets each
 * super-block's d. */
/* Gate/up weight formats: Q3_K (110-byte super-blocks of 256, one d per
 * super-block) or Q4_0 (18-byte blocks of 32, one d per block: dw[b]). */
#define GU_Q3K 0
#define GU_Q4_0 1
static int64_t gu_row_bytes(int fmt, int L) {
  return fmt == GU_Q4_0 ? (int64_t)(L / 32) * IQ4NL_BYTES : (int64_t)(L / Q3K_VALUES) * Q3K_BYTES;
}

static void gateup_row_dots_q4_0(const uint8_t* row, const uint8_t* act, int L, int32_t* I32, int32_t* I16,
                                 double* dw) {
  for (int b = 0; b < L / 32; ++b) {
    int8_t v[32];
    orc_q4_0_decode(row + (int64_t)b * IQ4NL_BYTES, v, &dw[b]);
    const int8_t* q = (const int8_t*)(act + (int64_t)b * Q81_BYTES + 4);
    int32_t acc32 = 0;
    for (int half = 0; half < 2; ++half) {
      int32_t acc16 = 0;
      for (int i = 0; i < 16; ++i) acc16 += (int32_t)v[half * 16 + i] * (int32_t)q[half * 16 + i];
      if (I16) I16[b * 2 + half] = acc16;
      acc32 += acc16;
    }
    I32[b] = acc32;
  }
}

static void gateup_row_dots(const uint8_t* row, const uint8_t* act, int L, int32_t* I32, int32_t* I16,
                            double* dw) {
  int nsb = L / Q3K_VALUES;
  for (int sb = 0; sb < nsb; ++sb) {
    int8_t v[Q3K_VALUES], sg[16];
    orc_q3k_decode(row + (int64_t)sb * Q3K_BYTES, v, sg, &dw[sb]);
    for (int bb = 0; bb < 8; ++bb) {
      int b = sb * 8 + bb;
      const int8_t* q = (const int8_t*)(act + (int64_t)b * Q81_BYTES + 4);
      int32_t acc32 = 0;
      for (int half = 0; half < 2; ++half) {
        int s = bb * 2 + half;
        int32_t acc16 = 0;
        for (int i = 0; i < 16; ++i) acc16 += (int32_t)v[bb * 32 + half * 16 + i] * (int32_t)q[half * 16 + i];
        if (I16) I16[b * 2 + half] = acc16;
        acc32 += (int32_t)sg[s] * acc16;
      }
      I32[b] = acc32;
    }
  }
}

/* Down block dots of one IQ4_NL (or Q4_0) row (F/32 blocks) against H (F/32
 * q8_1 blocks): J32[b] = sum_i K(i) * qH(i), K the block's integer weight
 * (table value, or nibble - 8); dd[b] gets each block's d. */
static void down_row_dots(int fmt, const uint8_t* row, const uint8_t* h, int F, int32_t* J32, double* dd) {
  int nb = F / IQ4NL_VALUES;
  for (int b = 0; b < nb; ++b) {
    int8_t kv[IQ4NL_VALUES];
    down_block_decode(fmt, row + (int64_t)b * IQ4NL_BYTES, kv, &dd[b]);
    const int8_t* q = (const int8_t*)(h + (int64_t)b * Q81_BYTES + 4);
    int32_t acc = 0;
    for (int i = 0; i < IQ4NL_VALUES; ++i) acc += (int32_t)kv[i] * (int32_t)q[i];
    J32[b] = acc;
  }
}

/* ------------------------------------------------------------------------ */
/* The expert stage, one pair at a time                                      */
/* ------------------------------------------------------------------------ */

/* One gate/up row r of expert weights gu_e against the token's q8_1 row, in
 * fp64: sum over blocks b (ascending) of dw[r][b/8] (Q3_K; dw[r][b] for Q4_0)
 * * dx[b] * I32[r][b].  I32, dw and dx are caller scratch of L/32 entries;
 * dx holds the activation block scales. */
static double gateup_row(int fmt, const uint8_t* xrow, const uint8_t* gu_e, int L, int r, int32_t* I32, double* dw,
                         const double* dx) {
  int nb = L / Q81_VALUES;
  int64_t row_bytes = gu_row_bytes(fmt, L);
  if (fmt == GU_Q4_0)
    gateup_row_dots_q4_0(gu_e + r * row_bytes, xrow, L, I32, NULL, dw);
  else
    gateup_row_dots(gu_e + r * row_bytes, xrow, L, I32, NULL, dw);
  double acc = 0.0;
  for (int b = 0; b < nb; ++b) acc += dw[fmt == GU_Q4_0 ? b : b / 8] * dx[b] * (double)I32[b];
  return acc;
}

/* Gate/up of one pair: G[F], U[F] in fp64 (rows 0..F-1 gate, F..2F-1 up). */
static void pair_gateup(int fmt, const uint8_t* xrow, const uint8_t* gu_e, int L, int F, double* G, double* U) {
  int nb = L / Q81_VALUES;
  int32_t* I32 = (int32_t*)malloc(sizeof(int32_t) * nb);
  double* dw = (double*)malloc(sizeof(double) * nb);  /* per super-block (Q3_K) or per block (Q4_0) */
  double* dx = (double*)malloc(sizeof(double) * nb);
  for (int b = 0; b < nb; ++b) dx[b] = orc_half_to_double(rd16(xrow + (int64_t)b * Q81_BYTES));
  for (int r = 0; r < 2 * F; ++r) {
    double acc = gateup_row(fmt, xrow, gu_e, L, r, I32, dw, dx);
    if (r < F) G[r] = acc;
    else U[r - F] = acc;
  }
  free(I32);
  free(dw);
  free(dx);
}

/* SwiGLU in fp64, then the q8_1 rounding of H (decision in fp32). */
static void pair_swiglu_q8_1(const double* G, const double* U, int F, uint8_t* hq) {
  float hv[Q81_VALUES];
  for (int b = 0; b < F / Q81_VALUES; ++b) {
    for (int i = 0; i < Q81_VALUES; ++i) {
      double g = G[b * Q81_VALUES + i], u = U[b * Q81_VALUES + i];
      double h = g / (1.0 + exp(-g)) * u;
      hv[i] = (float)h;
    }
    orc_q8_1_quantize_block(hv, hq + (int64_t)b * Q81_BYTES);
  }
}

/* Down of one pair: O[l] = sum_b dd[l][b] * dH[b] * J32[l][b], fp64. */
static void pair_down(int fmt, const uint8_t* hq, const uint8_t* dn_e, int L, int F, double* O) {
  int nb = F / IQ4NL_VALUES;
  int64_t row_bytes = (int64_t)nb * IQ4NL_BYTES;
  int32_t* J32 = (int32_t*)malloc(sizeof(int32_t) * nb);
  double* dd = (double*)malloc(sizeof(double) * nb);
  double* dh = (double*)malloc(sizeof(double) * nb);
  for (int b = 0; b < nb; ++b) dh[b] = orc_half_to_double(rd16(hq + (int64_t)b * Q81_BYTES));
  for (int l = 0; l < L; ++l) {
    down_row_dots(fmt, dn_e + l * row_bytes, hq, F, J32, dd);
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) acc += dd[b] * dh[b] * (double)J32[b];
    O[l] = acc;
  }
  free(J32);
  free(dd);
  free(dh);
}

/* Full stage for a list of tokens.
 *   x_q8     [T][L/32] q8_1         idx, w  [T][k]
 *   gateup   [E][2F][L/256] Q3_K    down    [E][L][F/32] IQ4_NL (down_fmt 0)
 *                                            or Q4_0 (down_fmt 1)
 *   tokens   the n_tok token ids to evaluate (NULL = all T, in order)
 *   y        [n_tok][L] fp64 (overwritten)
 *   h_out    [n_tok*k][F/32] q8_1 H per pair (NULL to skip); an invalid
 *            expert id leaves its H blocks all zero
 *   gu_out   [n_tok*k][2F] fp64 G then U per pair (NULL to skip)
 * Pairs with an expert id outside [0, E) contribute nothing.  Returns the
 * number of such pairs among the evaluated tokens. */
int64_t orc_forward_fmt(const uint8_t* x_q8, const int32_t* idx, const float* w, const uint8_t* gateup, int gu_fmt,
                        const uint8_t* down, int down_fmt, int64_t T, int L, int F, int E, int k,
                        const int64_t* tokens, int64_t n_tok, double* y, uint8_t* h_out, double* gu_out) {
  if (!tokens) n_tok = T;
  int64_t xrow_bytes = (int64_t)(L / Q81_VALUES) * Q81_BYTES;
  int64_t hrow_bytes = (int64_t)(F / Q81_VALUES) * Q81_BYTES;
  int64_t gu_e_bytes = (int64_t)2 * F * gu_row_bytes(gu_fmt, L);
  int64_t dn_e_bytes = (int64_t)L * (F / IQ4NL_VALUES) * IQ4NL_BYTES;
  int64_t dropped = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : dropped)
  for (int64_t it = 0; it < n_tok; ++it) {
    int64_t t = tokens ? tokens[it] : it;
    double* yt = y + it * L;
    double* G = (double*)malloc(sizeof(double) * F);
    double* U = (double*)malloc(sizeof(double) * F);
    double* O = (double*)malloc(sizeof(double) * L);
    uint8_t* hq = (uint8_t*)malloc(hrow_bytes);
    for (int l = 0; l < L; ++l) yt[l] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      int64_t po = it * k + j;
      if (e < 0 || e >= E) {
        ++dropped;
        if (h_out) memset(h_out + po * hrow_bytes, 0, hrow_bytes);
        if (gu_out)
          for (int f = 0; f < 2 * F; ++f) gu_out[po * 2 * F + f] = 0.0;
        continue;
      }
      pair_gateup(gu_fmt, x_q8 + t * xrow_bytes, gateup + e * gu_e_bytes, L, F, G, U);
      pair_swiglu_q8_1(G, U, F, hq);
      pair_down(down_fmt, hq, down + e * dn_e_bytes, L, F, O);
      double wj = (double)w[t * k + j];
      for (int l = 0; l < L; ++l) yt[l] += wj * O[l];
      if (h_out) memcpy(h_out + po * hrow_bytes, hq, hrow_bytes);
      if (gu_out) {
        memcpy(gu_out + po * 2 * F, G, sizeof(double) * F);
        memcpy(gu_out + po * 2 * F + F, U, sizeof(double) * F);
      }
    }
    free(G);
    free(U);
    free(O);
    free(hq);
  }
  return dropped;
}

int64_t orc_forward(const uint8_t* x_q8, const int32_t* idx, const float* w, const uint8_t* gateup,
                    const uint8_t* down, int64_t T, int L, int F, int E, int k, const int64_t* tokens,
                    int64_t n_tok, double* y, uint8_t* h_out, double* gu_out) {
  return orc_forward_fmt(x_q8, idx, w, gateup, GU_Q3K, down, DOWN_IQ4NL, T, L, F, E, k, tokens, n_tok, y, h_out,
                         gu_out);
}

/* Down projection and combine only, from given H (q8_1, [T*k][F/32] in pair
 * order): y[t] = sum_j w[t][j] * O(H[t*k+j]).  Used to check the second half
 * of the stage against a GPU's own H. */
void orc_down_combine_fmt(const uint8_t* h_q8, const int32_t* idx, const float* w, const uint8_t* down,
                          int down_fmt, int64_t T, int L, int F, int E, int k, const int64_t* tokens,
                          int64_t n_tok, double* y) {
  if (!tokens) n_tok = T;
  int64_t hrow_bytes = (int64_t)(F / Q81_VALUES) * Q81_BYTES;
  int64_t dn_e_bytes = (int64_t)L * (F / IQ4NL_VALUES) * IQ4NL_BYTES;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n_tok; ++it) {
    int64_t t = tokens ? tokens[it] : it;
    double* yt = y + it * L;
    double* O = (double*)malloc(sizeof(double) * L);
    for (int l = 0; l < L; ++l) yt[l] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      if (e < 0 || e >= E) continue;
      pair_down(down_fmt, h_q8 + (t * k + j) * hrow_bytes, down + e * dn_e_bytes, L, F, O);
      double wj = (double)w[t * k + j];
      for (int l = 0; l < L; ++l) yt[l] += wj * O[l];
    }
    free(O);
  }
}

void orc_down_combine(const uint8_t* h_q8, const int32_t* idx, const float* w, const uint8_t* down, int64_t T,
                      int L, int F, int E, int k, const int64_t* tokens, int64_t n_tok, double* y) {
  orc_down_combine_fmt(h_q8, idx, w, down, DOWN_IQ4NL, T, L, F, E, k, tokens, n_tok, y);
}

/* H of chosen 32-feature blocks, for checking H at sizes where the whole
 * stage is too slow: for i < n, the q8_1 block fb[i] of pair p = pair[i]'s H
 * (36 bytes at out + 36 i), that is G and U of features 32 fb .. 32 fb + 31
 * (gate/up rows f and F + f), SwiGLU and the q8_1 rounding -- the steps of
 * orc_forward_fmt for those 64 weight rows alone, so the bytes equal the
 * forward's H block.  Pairs with an expert id outside [0, E) give zeros. */
void orc_h_blocks_fmt(const uint8_t* x_q8, const int32_t* idx, const uint8_t* gateup, int gu_fmt, int64_t T, int L,
                      int F, int E, int k, int64_t n, const int64_t* pair, const int32_t* fb, uint8_t* out) {
  int nb = L / Q81_VALUES;
  int64_t xrow_bytes = (int64_t)nb * Q81_BYTES;
  int64_t gu_e_bytes = (int64_t)2 * F * gu_row_bytes(gu_fmt, L);
  (void)T;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < n; ++i) {
    int64_t p = pair[i];
    int e = idx[p];
    uint8_t* o = out + i * Q81_BYTES;
    if (e < 0 || e >= E) {
      memset(o, 0, Q81_BYTES);
      continue;
    }
    const uint8_t* xrow = x_q8 + (p / k) * xrow_bytes;
    int32_t* I32 = (int32_t*)malloc(sizeof(int32_t) * nb);
    double* dw = (double*)malloc(sizeof(double) * nb);
    double* dx = (double*)malloc(sizeof(double) * nb);
    double G[Q81_VALUES], U[Q81_VALUES];
    for (int b = 0; b < nb; ++b) dx[b] = orc_half_to_double(rd16(xrow + (int64_t)b * Q81_BYTES));
    for (int f = 0; f < Q81_VALUES; ++f) {
      int feat = fb[i] * Q81_VALUES + f;
      G[f] = gateup_row(gu_fmt, xrow, gateup + e * gu_e_bytes, L, feat, I32, dw, dx);
      U[f] = gateup_row(gu_fmt, xrow, gateup + e * gu_e_bytes, L, F + feat, I32, dw, dx);
    }
    pair_swiglu_q8_1(G, U, Q81_VALUES, o);
    free(I32);
    free(dw);
    free(dx);
  }
}

/* Integer block-dot probes.
 * Gate/up: for probe n = (pair p = t*k + j, row r < 2F): out32[n][L/32] = I32,
 * out16[n][L/16] = I16 (either may be NULL).  Down: for probe n = (pair p,
 * row l < L) with H given in pair order: out[n][F/32] = J32.  Probes whose
 * pair has an invalid expert id are filled with zeros. */
void orc_probe_gateup_fmt(const uint8_t* x_q8, const int32_t* idx, const uint8_t* gateup, int gu_fmt, int64_t T,
                          int L, int F, int E, int k, int64_t n, const int64_t* pair, const int32_t* row,
                          int32_t* out32, int32_t* out16) {
  int nb = L / Q81_VALUES;
  int64_t xrow_bytes = (int64_t)nb * Q81_BYTES;
  int64_t row_bytes = gu_row_bytes(gu_fmt, L);
  (void)T;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t p = pair[i];
    int e = idx[p];
    int32_t* o32 = out32 ? out32 + i * nb : NULL;
    int32_t* o16 = out16 ? out16 + i * 2 * nb : NULL;
    int32_t tmp32[L / Q81_VALUES];
    double dw[L / Q81_VALUES];
    if (e < 0 || e >= E) {
      if (o32) memset(o32, 0, sizeof(int32_t) * nb);
      if (o16) memset(o16, 0, sizeof(int32_t) * 2 * nb);
      continue;
    }
    const uint8_t* wrow = gateup + ((int64_t)e * 2 * F + row[i]) * row_bytes;
    if (gu_fmt == GU_Q4_0)
      gateup_row_dots_q4_0(wrow, x_q8 + (p / k) * xrow_bytes, L, tmp32, o16, dw);
    else
      gateup_row_dots(wrow, x_q8 + (p / k) * xrow_bytes, L, tmp32, o16, dw);
    if (o32) memcpy(o32, tmp32, sizeof(int32_t) * nb);
  }
}

void orc_probe_gateup(const uint8_t* x_q8, const int32_t* idx, const uint8_t* gateup, int64_t T, int L, int F,
                      int E, int k, int64_t n, const int64_t* pair, const int32_t* row, int32_t* out32,
                      int32_t* out16) {
  orc_probe_gateup_fmt(x_q8, idx, gateup, GU_Q3K, T, L, F, E, k, n, pair, row, out32, out16);
}

void orc_probe_down_fmt(const uint8_t* h_q8, const int32_t* idx, const uint8_t* down, int down_fmt, int64_t T,
                        int L, int F, int E, int k, int64_t n, const int64_t* pair, const int32_t* row,
                        int32_t* out) {
  int nb = F / IQ4NL_VALUES;
  int64_t hrow_bytes = (int64_t)nb * Q81_BYTES;
  int64_t row_bytes = (int64_t)nb * IQ4NL_BYTES;
  (void)T;
  (void)k;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t p = pair[i];
    int e = idx[p];
    double dd[F / IQ4NL_VALUES];
    if (e < 0 || e >= E) {
      memset(out + i * nb, 0, sizeof(int32_t) * nb);
      continue;
    }
    const uint8_t* wrow = down + ((int64_t)e * L + row[i]) * row_bytes;
    down_row_dots(down_fmt, wrow, h_q8 + p * hrow_bytes, F, out + i * nb, dd);
  }
}

void orc_probe_down(const uint8_t* h_q8, const int32_t* idx, const uint8_t* down, int64_t T, int L, int F, int E,
                    int k, int64_t n, const int64_t* pair, const int32_t* row, int32_t* out) {
  orc_probe_down_fmt(h_q8, idx, down, DOWN_IQ4NL, T, L, F, E, k, n, pair, row, out);
}

/* ------------------------------------------------------------------------ */
/* Latent D / U dense projections (Q8_0 weights x q8_1 activations)          */
/* ------------------------------------------------------------------------ */

/* Source: page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", the
 * lat_dense_w11.cu commit message: the two dense projections of a latent
 * layer (D into the latent rows, U back out of them) are Q8_0 x q8_1 integer
 * dots per 32-value block, and D rounds its products to the latent rows'
 * q8_1 blocks with the same rule as the stage's other q8_1 stores.
 *
 * Q8_0 (ggml): 32 weights in 34 bytes = d (fp16) | qs[32] (int8); weight
 * i = d * qs[i]. */
#define Q80_BYTES 34
#define Q80_VALUES 32

void orc_q8_0_decode(const uint8_t* blk, int8_t* q, double* d) {
  for (int i = 0; i < Q80_VALUES; ++i) q[i] = (int8_t)blk[2 + i];
  *d = orc_half_to_double(rd16(blk));
}
void orc_dequant_q8_0(const uint8_t* blocks, int64_t nblocks, double* out) {
  for (int64_t b = 0; b < nblocks; ++b) {
    int8_t q[Q80_VALUES];
    double d;
    orc_q8_0_decode(blocks + b * Q80_BYTES, q, &d);
    for (int i = 0; i < Q80_VALUES; ++i) out[b * Q80_VALUES + i] = d * (double)q[i];
  }
}

/* Projection weight formats: Q8_0, or Q4_0 (the PR page's section "Not done"
 * names a Q4_0 projection file; its block is the one orc_q4_0_decode reads,
 * 18 bytes per 32 weights). */
#define DENSE_Q8_0 0
#define DENSE_Q4_0 1
static int64_t dense_block_bytes(int fmt) { return fmt == DENSE_Q4_0 ? IQ4NL_BYTES : Q80_BYTES; }

/* Block dots of weight row w (K/32 Q8_0 or Q4_0 blocks) with activation row x
 * (K/32 q8_1 blocks): D32[b] = sum_i qw(i) * qx(i); dw[b], dx[b] get the
 * two block scales. */
static void dense_row_dots(int fmt, const uint8_t* w, const uint8_t* x, int K, int32_t* D32, double* dw,
                           double* dx) {
  int nb = K / Q80_VALUES;
  for (int b = 0; b < nb; ++b) {
    int8_t qw[Q80_VALUES], qx[Q81_VALUES];
    if (fmt == DENSE_Q4_0)
      orc_q4_0_decode(w + (int64_t)b * IQ4NL_BYTES, qw, &dw[b]);
    else
      orc_q8_0_decode(w + (int64_t)b * Q80_BYTES, qw, &dw[b]);
    orc_q8_1_decode(x + (int64_t)b * Q81_BYTES, qx, &dx[b]);
    int32_t acc = 0;
    for (int i = 0; i < Q80_VALUES; ++i) acc += (int32_t)qw[i] * (int32_t)qx[i];
    D32[b] = acc;
  }
}

/* y[t][n] = sum over blocks b (ascending) of dw[n][b] * dx[t][b] * D32[t][n][b]
 * in fp64, for the tokens tok[0..n_tok) (all T tokens when tok is NULL).
 * x [T][K/32] q8_1, w [N][K/32] Q8_0 (fmt 0) or Q4_0 (fmt 1), y [n_tok][N]. */
void orc_dense_fmt(const uint8_t* x_q8, int64_t T, const uint8_t* w, int fmt, int N, int K, const int64_t* tok,
                   int64_t n_tok, double* y) {
  int nb = K / Q80_VALUES;
  int64_t xrow = (int64_t)nb * Q81_BYTES, wrow = (int64_t)nb * dense_block_bytes(fmt);
  (void)T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_tok; ++i) {
    int64_t t = tok ? tok[i] : i;
    int32_t* D32 = (int32_t*)malloc(sizeof(int32_t) * nb);
    double* dw = (double*)malloc(sizeof(double) * nb);
    double* dx = (double*)malloc(sizeof(double) * nb);
    for (int n = 0; n < N; ++n) {
      dense_row_dots(fmt, w + n * wrow, x_q8 + t * xrow, K, D32, dw, dx);
      double acc = 0.0;
      for (int b = 0; b < nb; ++b) acc += dw[b] * dx[b] * (double)D32[b];
      y[i * N + n] = acc;
    }
    free(D32);
    free(dw);
    free(dx);
  }
}

void orc_dense_q8_0(const uint8_t* x_q8, int64_t T, const uint8_t* w, int N, int K, const int64_t* tok,
                    int64_t n_tok, double* y) {
  orc_dense_fmt(x_q8, T, w, DENSE_Q8_0, N, K, tok, n_tok, y);
}

/* Dense block-dot probes: for probe i = (token tok[i], weight row row[i]),
 * out[i][K/32] = D32. */
void orc_probe_dense_fmt(const uint8_t* x_q8, int64_t T, const uint8_t* w, int fmt, int N, int K, int64_t n,
                         const int64_t* tok, const int32_t* row, int32_t* out) {
  int nb = K / Q80_VALUES;
  int64_t xrow = (int64_t)nb * Q81_BYTES, wrow = (int64_t)nb * dense_block_bytes(fmt);
  (void)T;
  (void)N;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double* dw = (double*)malloc(sizeof(double) * nb);
    double* dx = (double*)malloc(sizeof(double) * nb);
    dense_row_dots(fmt, w + row[i] * wrow, x_q8 + tok[i] * xrow, K, out + i * nb, dw, dx);
    free(dw);
    free(dx);
  }
}

void orc_probe_dense(const uint8_t* x_q8, int64_t T, const uint8_t* w, int N, int K, int64_t n, const int64_t* tok,
                     const int32_t* row, int32_t* out) {
  orc_probe_dense_fmt(x_q8, T, w, DENSE_Q8_0, N, K, n, tok, row, out);
}

/* ------------------------------------------------------------------------ */
/* Router: softmax over the experts, top-k, renormalised weights             */
/* ------------------------------------------------------------------------ */

/* Source: page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section
 * "Contents" and the HIP backend page (the MoE router picks the top experts of
 * each token and the stage combines their outputs with the router's weights);
 * the task's workloads state the rule: softmax over E, top-k, renormalised.
 *
 * For each token t:  p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l)  (fp64);
 * the k experts of largest p, taken in descending order, equal probabilities
 * (equal logits) in ascending expert order; w_j = p_(j) / sum_i p_(i) over the
 * k picks (fp64), stored as fp32.  The ranking is made on the logits: softmax
 * is strictly increasing in the logit, and ranking the logits keeps that order
 * where fp64 exp would round distinct tiny probabilities to the same value.
 * A row needs at least one finite logit; -inf logits (masked experts) have
 * p = 0 and are picked only when fewer than k logits are finite. */
void orc_router_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e)
      if ((double)l[e] > mx) mx = (double)l[e];
    double* p = (double*)malloc(sizeof(double) * E);
    unsigned char* taken = (unsigned char*)calloc(E, 1);
    double den = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - mx);
      den += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= den;
    double sel = 0.0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower index */
      }
      taken[best] = 1;
      idx[t * k + j] = best;
      sel += p[best];
    }
    for (int j = 0; j < k; ++j) w[t * k + j] = (float)(p[idx[t * k + j]] / sel);
    free(p);
    free(taken);
  }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
