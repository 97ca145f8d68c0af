/*
 * stepq_oracle.c -- CPU oracle for the STEPQuant packed-state decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow executable specification that the
 * GPU library is checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  The product library neither links nor calls it, and this file
 * includes nothing from the product.
 *
 * What it follows (page: "STEPQuant" paper digest, vibe-research silicon-writer readme):
 *   - Background, "linear attention only changes the memory bill": a head keeps a d_k x d_v state
 *     that every step updates from key, value and retention gate and reads out with the query.
 *   - Background, "why plain INT8 is still not stable": each decode step dequantizes, updates and
 *     requantizes the state; A_t holds both the retention gate and the delta update.
 *   - Method 3, "Key-Row-Aware Dual-Axis Fitting": X_hat[i,j] = r_i * c_j * z[i,j]; r_i grows with
 *     the row's mean magnitude and gives high-omega rows finer steps; c_j is an omega-weighted MSE
 *     fit over value columns with r fixed; z are low-bit integers stored per the offline map.
 *   - Method 4, "the execution path of each decode step": reconstruct from codes, scales and FP16
 *     pivots; retention + delta update + readout on the float tile; the output leaves before
 *     requantization; refit r and c; pack codes and scales with pivots kept in FP16.
 * The scale formulas (r_i = (mean_j|S_ij| + 1e-8)/(1 + omega_i/mean omega), c_j initialised to
 * max_i|S_ij/r_i|/qmax, one omega-weighted least-squares refit with z fixed, symmetric
 * round-half-even with qmax = 2^(b-1)-1) and the gate A_t = Diag(a)(I - beta k k^T) are the
 * readings taken here where the pages leave the step open; the other gate order,
 * A_t = (I - beta k k^T) Diag(a), is available as a plan option (ORC_DECAY_FIRST).
 *
 * This is one binary32 evaluation order of that step, fixed so that a GPU can follow it bit for
 * bit; oracle/plain.py states the step in binary64 without it, and the tests check this file
 * against that statement within the binary32 error bounds.  The order's choices:
 *   - the stored state is a row factor f_i (r_hat_i, or 1 on FP16 pivot rows) times
 *     X_ij = c_j z_ij (exact) or the pivot value;
 *   - the updated state is kept as S_ij = M_i T_ij with T_ij = fma(K_i, e_ij, X_ij),
 *     M_i = a_i f_i and K_i = (beta k_i) / M_i, which is a_i f_i X_ij + beta k_i e_ij;
 *     a row whose gate is below 2^-72 in magnitude (its previous state is erased) takes
 *     X_ij := 0, and such a row or one with f_i = 0 takes M_i = beta k_i, K_i = 1;
 *   - every later per-row scale (readout coefficient q_i M_i, row magnitude |M_i|, the scaled
 *     state y = T (M_i / r_hat_i)) is one per-row product;
 *   - r_i = (mean + 1e-8) * (1 / den_i) with the reciprocal taken once per plan;
 *   - codes round the exact product y * (1/c) once (no intermediate rounding of the product).
 * Arithmetic: IEEE binary32, round to nearest even, subnormals kept.  Every operation is rounded
 * on its own; a fused multiply-add appears only where fmaf() is written.  Build with
 * -ffp-contract=off and without -ffast-math.  Sums run in a fixed order:
 *   tree(x_0..x_{n-1})  pairwise: tree(first half) + tree(second half); tree(x) = x.
 *   dot(x, y)           consecutive blocks of 32 terms are each accumulated first to last with
 *                       fused multiply-adds (the first term a rounded product), and the block
 *                       sums are combined by tree().
 * The two fixed orders make CPU and GPU results comparable bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FLAG_NONFINITE 1u   /* a row of the updated state is not finite        */
#define ORC_FLAG_SCALE_OVF 2u   /* a row or column factor overflowed binary16      */
#define ORC_FLAG_PIVOT_OVF 4u   /* an FP16 pivot entry overflowed binary16         */

#define ORC_LANES 64            /* column owners of the packed code layout         */

/* ------------------------------------------------------------------------------------------ */
/* binary16 conversion, written from the IEEE 754 definition                                  */
/* ------------------------------------------------------------------------------------------ */

uint16_t orc_f32_to_f16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t ex = (u >> 23) & 0xFFu;
  uint32_t man = u & 0x7FFFFFu;
  if (ex == 0xFFu) return (uint16_t)(sign | (man ? (0x7E00u | (man >> 13)) : 0x7C00u));
  if (ex == 0u) return (uint16_t)sign; /* binary32 subnormals are far below half of 2^-24 */
  int e = (int)ex - 127;
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  uint32_t sig = man | 0x800000u; /* 24 significant bits */
  if (e >= -14) {                 /* lands in the binary16 normal range */
    uint32_t qv = sig >> 13, rem = sig & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (qv & 1u))) qv++;
    /* qv in [0x400, 0x800]; a carry into 0x800 bumps the exponent, 0x7C00 being infinity */
    return (uint16_t)(sign | (((uint32_t)(e + 15) << 10) + (qv - 0x400u)));
  }
  int sh = -e - 1; /* value / 2^-24 = sig * 2^(e+1) */
  if (sh > 24) return (uint16_t)sign;
  uint32_t qv = sig >> sh, rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (rem > half || (rem == half && (qv & 1u))) qv++;
  return (uint16_t)(sign | qv);
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t ex = (h >> 10) & 0x1Fu, man = h & 0x3FFu, u;
  if (ex == 0x1Fu) {
    u = sign | 0x7F800000u | (man << 13);
  } else if (ex == 0u) {
    float f = (float)man * 0x1p-24f; /* exact: man < 2^10 */
    return sign ? -f : f;
  } else {
    u = sign | ((ex + 112u) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------------------------------ */
/* fixed-order reductions                                                                     */
/* ------------------------------------------------------------------------------------------ */

static float tree_sum(const float* x, int n) {
  if (n == 1) return x[0];
  return tree_sum(x, n / 2) + tree_sum(x + n / 2, n - n / 2);
}

#define ORC_BLOCK 32      /* rows of one fma chain in dot() */

/* dot over n >= 1 terms, x[i*xs], y[i*ys]: blocks of 32 consecutive terms (the last one
   shorter if 32 does not divide n), at most 16 blocks */
static float dot_fixed(const float* x, int xs, const float* y, int ys, int n) {
  float blk[16];
  int nb = (n + ORC_BLOCK - 1) / ORC_BLOCK;
  for (int m = 0; m < nb; m++) {
    int i0 = ORC_BLOCK * m, i1 = i0 + ORC_BLOCK < n ? i0 + ORC_BLOCK : n;
    float s = x[i0 * xs] * y[i0 * ys];
    for (int i = i0 + 1; i < i1; i++) s = fmaf(x[i * xs], y[i * ys], s);
    blk[m] = s;
  }
  return tree_sum(blk, nb);
}

float orc_tree_sum(const float* x, int n) { return tree_sum(x, n); }
float orc_dot(const float* x, const float* y, int n) { return dot_fixed(x, 1, y, 1, n); }

static float rcp0(float x) { return x == 0.0f ? 0.0f : 1.0f / x; }

/* round half to even of the exact product a*b (binary32 operands: the product is exact in
   binary64), as a binary64 value */
static double rne_prod(float a, float b) { return nearbyint((double)a * (double)b); }

static double clampd(double x, double lo, double hi) { return x < lo ? lo : (x > hi ? hi : x); }

/* ------------------------------------------------------------------------------------------ */
/* packed segment layout of one head                                                          */
/*                                                                                            */
/*   code block   lane L (0..63) owns columns G*L .. G*L+G-1, G = d_v/64.  Its bit stream     */
/*                holds, for every non-pivot row in ascending order, the G codes of that row  */
/*                in column order, b_i bits each, two's complement, least significant bit     */
/*                first; the stream is padded with zero bits to D whole 32-bit words.  Word   */
/*                w of lane L sits at byte 4*(64*w + L).  Block size 256*D bytes.             */
/*   pivot block  every pivot row in ascending order, d_v binary16 values.                    */
/*   r block      d_k binary16 row factors (0 for pivot rows)     -- absent if all rows pivot */
/*   c block      d_v binary16 column factors                     -- absent if all rows pivot */
/*   the segment is padded to a multiple of 256 bytes.                                        */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int dk, dv, G, npiv, allpiv;
  long words;       /* D */
  long off_piv, off_r, off_c, bytes;
  long rowpos[256]; /* stream bit offset of the first code of each non-pivot row */
} seg_layout;

static seg_layout layout_of(int dk, int dv, const int8_t* bits, const uint8_t* pivot) {
  seg_layout s;
  s.dk = dk;
  s.dv = dv;
  s.G = dv / ORC_LANES;
  s.npiv = 0;
  long lane_bits = 0;
  for (int i = 0; i < dk; i++) {
    s.rowpos[i] = lane_bits;
    if (pivot[i]) s.npiv++;
    else lane_bits += (long)s.G * bits[i];
  }
  s.allpiv = (s.npiv == dk);
  s.words = (lane_bits + 31) / 32;
  s.off_piv = 256L * s.words;
  s.off_r = s.off_piv + 2L * dv * s.npiv;
  s.off_c = s.off_r + (s.allpiv ? 0 : 2L * dk);
  long end = s.off_c + (s.allpiv ? 0 : 2L * dv);
  s.bytes = (end + 255) / 256 * 256;
  return s;
}

long orc_segment_bytes(int dk, int dv, const int8_t* bits, const uint8_t* pivot) {
  return layout_of(dk, dv, bits, pivot).bytes;
}

/* stream bit position of code (i, j) for a non-pivot row i */
static long code_bitpos(const seg_layout* s, const int8_t* bits, int i, int j) {
  return s->rowpos[i] + (long)(j % s->G) * bits[i];
}

static int stream_bit(const uint8_t* seg, int lane, long p) {
  long w = p / 32;
  int t = (int)(p % 32);
  uint32_t word;
  memcpy(&word, seg + 4 * (ORC_LANES * w + lane), 4);
  return (int)((word >> t) & 1u);
}

static void set_stream_bit(uint8_t* seg, int lane, long p, int v) {
  long w = p / 32;
  int t = (int)(p % 32);
  uint32_t word;
  memcpy(&word, seg + 4 * (ORC_LANES * w + lane), 4);
  word = (word & ~(1u << t)) | ((uint32_t)(v & 1) << t);
  memcpy(seg + 4 * (ORC_LANES * w + lane), &word, 4);
}

static int get_code(const seg_layout* s, const uint8_t* seg, const int8_t* bits, int i, int j) {
  long p = code_bitpos(s, bits, i, j);
  int b = bits[i], lane = j / s->G, v = 0;
  for (int t = 0; t < b; t++) v |= stream_bit(seg, lane, p + t) << t;
  if (v & (1 << (b - 1))) v -= 1 << b; /* two's complement */
  return v;
}

static void put_code(const seg_layout* s, uint8_t* seg, const int8_t* bits, int i, int j,
                     int z) {
  long p = code_bitpos(s, bits, i, j);
  int b = bits[i], lane = j / s->G;
  uint32_t v = (uint32_t)z & ((1u << b) - 1u);
  for (int t = 0; t < b; t++) set_stream_bit(seg, lane, p + t, (int)((v >> t) & 1u));
}

static int pivot_index(const uint8_t* pivot, int i) {
  int n = 0;
  for (int r = 0; r < i; r++) n += pivot[r] ? 1 : 0;
  return n;
}

static uint16_t rd16(const uint8_t* p) {
  uint16_t h;
  memcpy(&h, p, 2);
  return h;
}

static void wr16(uint8_t* p, uint16_t h) { memcpy(p, &h, 2); }

/* ------------------------------------------------------------------------------------------ */
/* decode (Method 3 reconstruction, Method 4 step 1)                                          */
/* ------------------------------------------------------------------------------------------ */

/* S_hat[i*dv+j] = r_i c_j z_ij rounded once (both two-factor products are exact, so the order of
   the two multiplications does not matter); pivot rows return their binary16 values.
   r16/c16/z may be NULL. Returns 0 or -1 if a code reads -2^(b-1), which the packer never
   writes. */
int orc_unpack(int dk, int dv, const int8_t* bits, const uint8_t* pivot, const uint8_t* seg,
               float* S_hat, uint16_t* r16, uint16_t* c16, int8_t* z) {
  seg_layout s = layout_of(dk, dv, bits, pivot);
  int bad = 0;
  for (int i = 0; i < dk; i++) {
    if (pivot[i]) {
      const uint8_t* row = seg + s.off_piv + 2L * dv * pivot_index(pivot, i);
      for (int j = 0; j < dv; j++) {
        S_hat[(long)i * dv + j] = orc_f16_to_f32(rd16(row + 2L * j));
        if (z) z[(long)i * dv + j] = 0;
      }
      if (r16) r16[i] = 0;
      continue;
    }
    float r = orc_f16_to_f32(rd16(seg + s.off_r + 2L * i));
    if (r16) r16[i] = rd16(seg + s.off_r + 2L * i);
    for (int j = 0; j < dv; j++) {
      int zi = get_code(&s, seg, bits, i, j);
      if (zi == -(1 << (bits[i] - 1))) bad = 1;
      float c = orc_f16_to_f32(rd16(seg + s.off_c + 2L * j));
      S_hat[(long)i * dv + j] = r * (c * (float)zi);
      if (z) z[(long)i * dv + j] = (int8_t)zi;
    }
  }
  if (c16)
    for (int j = 0; j < dv; j++) c16[j] = s.allpiv ? 0 : rd16(seg + s.off_c + 2L * j);
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------------------------ */
/* requantize and pack (Method 3 fitting, Method 4 steps 4-5)                                 */
/* ------------------------------------------------------------------------------------------ */

/* plan-time denominators den_i = 1 + omega_i / mean(omega); 1 when the mean is zero */
void orc_row_den(int dk, const float* omega, float* den) {
  float mean = tree_sum(omega, dk) * (1.0f / (float)dk);
  for (int i = 0; i < dk; i++) den[i] = mean > 0.0f ? 1.0f + omega[i] / mean : 1.0f;
}

/* Requantize the state S_ij = M_i T_ij (dk x dv row-major T, per-row M) into seg.
   pre (optional, dk*dv) receives the final pre-rounding value y_ij * (1/c_j) (exact, binary64)
   of every quantized entry (0 elsewhere), z0_out (optional, dk*dv) the first codes (0 on pivot
   and dead rows), c0_out (optional, dv) the first column factors. */
static int requant(int dk, int dv, const int8_t* bits, const uint8_t* pivot, const float* omega,
                   const float* T, const float* M, uint8_t* seg, double* pre, int8_t* z0_out,
                   float* c0_out, uint32_t* flags) {
  seg_layout s = layout_of(dk, dv, bits, pivot);
  uint32_t fl = 0;
  float* den = (float*)malloc(sizeof(float) * dk);
  float* ir = (float*)malloc(sizeof(float) * dk);
  float* W = (float*)malloc(sizeof(float) * dk);
  float* qmax = (float*)malloc(sizeof(float) * dk);
  float* iq = (float*)malloc(sizeof(float) * dk);
  float* absrow = (float*)malloc(sizeof(float) * dv);
  float* y = (float*)malloc(sizeof(float) * dk * dv);
  float* z0 = (float*)malloc(sizeof(float) * dk * dv);
  float* a = (float*)malloc(sizeof(float) * dk * dv);
  float* c0 = (float*)malloc(sizeof(float) * dv);
  float* ic = (float*)malloc(sizeof(float) * dv);
  orc_row_den(dk, omega, den);
  memset(seg, 0, (size_t)s.bytes);

  /* row factor r_i = (mean_j |S_ij| + 1e-8) / den_i with mean_j |S_ij| = |M_i| mean_j |T_ij|,
     stored as binary16; the division is a product with the plan's reciprocal 1/den_i */
  for (int i = 0; i < dk; i++) {
    for (int j = 0; j < dv; j++) absrow[j] = fabsf(T[(long)i * dv + j]);
    float m = (tree_sum(absrow, dv) * fabsf(M[i])) * (1.0f / (float)dv);
    if (!isfinite(m)) fl |= ORC_FLAG_NONFINITE;
    qmax[i] = pivot[i] ? 0.0f : (float)((1 << (bits[i] - 1)) - 1);
    iq[i] = pivot[i] ? 0.0f : 1.0f / qmax[i];
    if (pivot[i]) { /* FP16 pivot row: the state value M_i T_ij stored raw, left out of the fit */
      uint8_t* row = seg + s.off_piv + 2L * dv * pivot_index(pivot, i);
      for (int j = 0; j < dv; j++) {
        uint16_t h = orc_f32_to_f16(M[i] * T[(long)i * dv + j]);
        if ((h & 0x7FFFu) == 0x7C00u) fl |= ORC_FLAG_PIVOT_OVF;
        wr16(row + 2L * j, h);
      }
      ir[i] = 0.0f;
      W[i] = 0.0f;
      continue;
    }
    float r = (m + 1e-8f) * (1.0f / den[i]);
    uint16_t rh = orc_f32_to_f16(r);
    if ((rh & 0x7FFFu) == 0x7C00u) fl |= ORC_FLAG_SCALE_OVF;
    wr16(seg + s.off_r + 2L * i, rh);
    float rr = orc_f16_to_f32(rh);
    ir[i] = rcp0(rr); /* a row whose factor rounds to zero is dead: all its codes are 0 */
    W[i] = (omega[i] * rr) * rr;
  }
  if (s.allpiv) {
    if (z0_out) memset(z0_out, 0, (size_t)dk * dv);
    if (c0_out) memset(c0_out, 0, sizeof(float) * dv);
    goto done;
  }

  /* y = S / r_hat = T_ij * (M_i * (1/r_hat_i)); c0_j = max_i |y_ij| / qmax_i */
  for (int i = 0; i < dk; i++) {
    float rho = M[i] * ir[i];
    for (int j = 0; j < dv; j++) y[(long)i * dv + j] = T[(long)i * dv + j] * rho;
  }
  for (int j = 0; j < dv; j++) {
    float mx = 0.0f;
    for (int i = 0; i < dk; i++) {
      float t = fabsf(y[(long)i * dv + j]) * iq[i];
      if (t > mx) mx = t;
    }
    c0[j] = mx;
    if (c0_out) c0_out[j] = mx;
  }
  /* first quantization with c0 (its clamp never binds: |y| / qmax <= c0), then the
     omega-weighted least-squares column refit:
     c1_j = argmin_c sum_i omega_i (S_ij - r_i c z0_ij)^2
          = sum_i W_i z0_ij y_ij / sum_i W_i z0_ij^2   with W_i = omega_i r_i^2, y = S / r */
  for (int j = 0; j < dv; j++) {
    float ic0 = rcp0(c0[j]);
    for (int i = 0; i < dk; i++) {
      long e = (long)i * dv + j;
      z0[e] = (float)clampd(rne_prod(y[e], ic0), -qmax[i], qmax[i]);
      /* NaN only follows a non-finite state (flagged); its debug copy reads 0 */
      if (z0_out) z0_out[e] = z0[e] == z0[e] ? (int8_t)z0[e] : 0;
      a[e] = W[i] * z0[e];
    }
    float num = dot_fixed(a + j, dv, y + j, dv, dk);
    float sq = dot_fixed(a + j, dv, z0 + j, dv, dk);
    float c1 = sq > 0.0f ? num / sq : c0[j];
    uint16_t ch = orc_f32_to_f16(c1);
    if ((ch & 0x7FFFu) == 0x7C00u) fl |= ORC_FLAG_SCALE_OVF;
    wr16(seg + s.off_c + 2L * j, ch);
    ic[j] = rcp0(orc_f16_to_f32(ch));
  }
  /* final symmetric round-half-even requantization with the refitted column factors */
  for (int i = 0; i < dk; i++) {
    if (pivot[i]) continue;
    for (int j = 0; j < dv; j++) {
      long e = (long)i * dv + j;
      if (pre) pre[e] = (double)y[e] * (double)ic[j];
      double zr = clampd(rne_prod(y[e], ic[j]), -qmax[i], qmax[i]);
      int zi = zr == zr ? (int)zr : 0; /* NaN only follows a non-finite state (flagged) */
      put_code(&s, seg, bits, i, j, zi);
    }
  }
done:
  if (pre)
    for (int i = 0; i < dk; i++)
      if (pivot[i])
        for (int j = 0; j < dv; j++) pre[(long)i * dv + j] = 0.0f;
  free(den); free(ir); free(W); free(qmax); free(iq); free(absrow);
  free(y); free(z0); free(a); free(c0); free(ic);
  if (flags) *flags |= fl;
  return 0;
}

/* Encode the fp32 state S (dk x dv row-major) into seg: the requantization of S = 1 * S.
   pre, z0_out, c0_out as for requant(). */
int orc_encode_dbg(int dk, int dv, const int8_t* bits, const uint8_t* pivot, const float* omega,
                   const float* S, uint8_t* seg, double* pre, int8_t* z0_out, float* c0_out,
                   uint32_t* flags) {
  float* one = (float*)malloc(sizeof(float) * dk);
  for (int i = 0; i < dk; i++) one[i] = 1.0f;
  int rc = requant(dk, dv, bits, pivot, omega, S, one, seg, pre, z0_out, c0_out, flags);
  free(one);
  return rc;
}

int orc_encode(int dk, int dv, const int8_t* bits, const uint8_t* pivot, const float* omega,
               const float* S, uint8_t* seg, double* pre, uint32_t* flags) {
  return orc_encode_dbg(dk, dv, bits, pivot, omega, S, seg, pre, NULL, NULL, flags);
}

/* ------------------------------------------------------------------------------------------ */
/* the decode step (Method 4)                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* Gate orders of A_t (both readings of the digest's "A_t contains the retention gate and the
   Delta update"):
     ORC_DELTA_FIRST  A = Diag(a)(I - beta k k^T): the delta update, then the decay of each row
                      (the literal reading; S_t = a_i (S - beta k u^T)_i + beta k_i v^T with
                      u = S^T k);
     ORC_DECAY_FIRST  A = (I - beta k k^T) Diag(a): the rows decay first and the delta update sees
                      the decayed state (u = (Diag(a) S)^T k, e = v - u, one e per column).
   For a scalar gate (GDN) the two are the same map; their binary32 results differ in rounding. */
#define ORC_DELTA_FIRST 0
#define ORC_DECAY_FIRST 1
#define ORC_GATE_ERASE 0x1p-72f   /* a gate below this erases the row's previous state */

/* One gated delta step on a tile given as per-row factors f_i (r_hat_i of a quantized row, 1 for a
   pivot row or an unquantized state) times X (c_j z_ij, exact; or the pivot / fp32 values), so
   that the stored state is f_i X_ij:
     u_j = dot_i(kc_i, X_ij)     kc_i = k_i f_i, or k_i (a_i f_i) when the rows decay first
     e_ij = fma(-a_i, u_j, v_j), or v_j - u_j when the rows decay first
     T_ij = fma(K_i, e_ij, X_ij),  and the updated state is S_ij = M_i T_ij with
     M_i = a_i f_i, K_i = (beta k_i) / M_i  (so M_i T_ij = a_i f_i X_ij + beta k_i e_ij)
   which is S <- A S + beta k v^T with A = Diag(a)(I - beta k k^T) (GDN: every a_i = alpha), or
   A = (I - beta k k^T) Diag(a).  A row with |a_i| < 2^-72 has its X row zeroed after u (its
   previous state is erased: S = beta k_i e); such a row and a dead one (f_i = 0) take M_i =
   beta k_i, K_i = 1.  out_j = dot_i(q_i M_i, T_ij).  T is updated in place (it holds X on
   entry). */
static void update_factored(int dk, int dv, float* T, float* M, const float* f, const float* q,
                            const float* k, const float* v, const float* a, float beta,
                            float* out, int order) {
  float* u = (float*)malloc(sizeof(float) * dv);
  float* kc = (float*)malloc(sizeof(float) * dk);
  float* K = (float*)malloc(sizeof(float) * dk);
  float* qm = (float*)malloc(sizeof(float) * dk);
  for (int i = 0; i < dk; i++) {
    float m = a[i] * f[i], bk = beta * k[i];
    kc[i] = order == ORC_DECAY_FIRST ? k[i] * m : k[i] * f[i];
    int erased = fabsf(a[i]) < ORC_GATE_ERASE;
    if (erased || f[i] == 0.0f) {
      M[i] = bk;
      K[i] = 1.0f;
    } else {
      M[i] = m;
      K[i] = bk / m;
    }
    qm[i] = q[i] * M[i];
  }
  for (int j = 0; j < dv; j++) u[j] = dot_fixed(kc, 1, T + j, dv, dk);
  for (int i = 0; i < dk; i++) {
    int erased = fabsf(a[i]) < ORC_GATE_ERASE;
    for (int j = 0; j < dv; j++) {
      long e = (long)i * dv + j;
      float ev = order == ORC_DECAY_FIRST ? v[j] - u[j] : fmaf(-a[i], u[j], v[j]);
      T[e] = fmaf(K[i], ev, erased ? 0.0f : T[e]);
    }
  }
  for (int j = 0; j < dv; j++) out[j] = dot_fixed(qm, 1, T + j, dv, dk);
  free(u); free(kc); free(K); free(qm);
}

/* Splits a segment into per-row factors f (r_hat, or 1 on pivot rows) and X = c_j z_ij (exact)
   or the pivot row's binary16 values.  Returns -1 on a corrupt code. */
static int decode_factored(int dk, int dv, const int8_t* bits, const uint8_t* pivot,
                           const uint8_t* seg, float* X, float* f) {
  int8_t* z = (int8_t*)malloc((size_t)dk * dv);
  float* Sh = (float*)malloc(sizeof(float) * dk * dv);
  uint16_t* r16 = (uint16_t*)malloc(sizeof(uint16_t) * dk);
  uint16_t* c16 = (uint16_t*)malloc(sizeof(uint16_t) * dv);
  int rc = orc_unpack(dk, dv, bits, pivot, seg, Sh, r16, c16, z);
  for (int i = 0; i < dk; i++) {
    f[i] = pivot[i] ? 1.0f : orc_f16_to_f32(r16[i]);
    for (int j = 0; j < dv; j++) {
      long e = (long)i * dv + j;
      X[e] = pivot[i] ? Sh[e] : orc_f16_to_f32(c16[j]) * (float)z[e];
    }
  }
  free(z); free(Sh); free(r16); free(c16);
  return rc;
}

/* Decode step of one (request, head) tile, in place on seg.  a has dk entries (all equal for
   GDN).  S_upd (optional) receives the updated state M_i T_ij rounded to binary32, pre
   (optional) the final pre-rounding values.  Returns 0, or -1 on a corrupt code. */
int orc_tile_step_dbg(int dk, int dv, const int8_t* bits, const uint8_t* pivot,
                      const float* omega, uint8_t* seg, const float* q, const float* k,
                      const float* v, const float* a, float beta, float* out, float* S_upd,
                      double* pre, int8_t* z0_out, float* c0_out, uint32_t* flags, int order) {
  float* T = (float*)calloc((size_t)dk * dv, sizeof(float));
  float* f = (float*)calloc((size_t)dk, sizeof(float));
  float* M = (float*)calloc((size_t)dk, sizeof(float));
  int rc = decode_factored(dk, dv, bits, pivot, seg, T, f);
  update_factored(dk, dv, T, M, f, q, k, v, a, beta, out, order);
  if (S_upd)
    for (int i = 0; i < dk; i++)
      for (int j = 0; j < dv; j++) S_upd[(long)i * dv + j] = M[i] * T[(long)i * dv + j];
  requant(dk, dv, bits, pivot, omega, T, M, seg, pre, z0_out, c0_out, flags);
  free(T);
  free(f);
  free(M);
  return rc;
}

int orc_tile_step_o(int dk, int dv, const int8_t* bits, const uint8_t* pivot,
                    const float* omega, uint8_t* seg, const float* q, const float* k,
                    const float* v, const float* a, float beta, float* out, float* S_upd,
                    double* pre, uint32_t* flags, int order) {
  return orc_tile_step_dbg(dk, dv, bits, pivot, omega, seg, q, k, v, a, beta, out, S_upd, pre,
                           NULL, NULL, flags, order);
}

int orc_tile_step(int dk, int dv, const int8_t* bits, const uint8_t* pivot, const float* omega,
                  uint8_t* seg, const float* q, const float* k, const float* v, const float* a,
                  float beta, float* out, float* S_upd, double* pre, uint32_t* flags) {
  return orc_tile_step_o(dk, dv, bits, pivot, omega, seg, q, k, v, a, beta, out, S_upd, pre,
                         flags, ORC_DELTA_FIRST);
}

/* FP32-state mode: the same update and readout on an unquantized state (warm-up, drift); the
   state is stored back as M_i T_ij rounded to binary32. */
void orc_fp32_step_o(int dk, int dv, float* S, const float* q, const float* k, const float* v,
                     const float* a, float beta, float* out, int order) {
  float* f = (float*)calloc((size_t)dk, sizeof(float));
  float* M = (float*)calloc((size_t)dk, sizeof(float));
  for (int i = 0; i < dk; i++) f[i] = 1.0f;
  update_factored(dk, dv, S, M, f, q, k, v, a, beta, out, order);
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) S[(long)i * dv + j] = M[i] * S[(long)i * dv + j];
  free(f);
  free(M);
}

void orc_fp32_step(int dk, int dv, float* S, const float* q, const float* k, const float* v,
                   const float* a, float beta, float* out) {
  orc_fp32_step_o(dk, dv, S, q, k, v, a, beta, out, ORC_DELTA_FIRST);
}

/* ------------------------------------------------------------------------------------------ */
/* batch helpers (plain loops over the functions above)                                       */
/* ------------------------------------------------------------------------------------------ */

void orc_f32_to_f16_n(const float* x, uint16_t* h, long n) {
  for (long i = 0; i < n; i++) h[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_n(const uint16_t* h, float* x, long n) {
  for (long i = 0; i < n; i++) x[i] = orc_f16_to_f32(h[i]);
}

/* T fp32-state steps on ntiles independent tiles.  Tile t, step s reads q/k/v at
   base + s*step_stride + t*dv (and a at a + s*a_step + t*dk, beta at beta[s*nt + t]) and writes
   out (if not NULL) likewise. */
void orc_fp32_run_o(int dk, int dv, int ntiles, int T, float* S, const float* q,
                    const float* k, const float* v, long step_stride, const float* a,
                    long a_step, const float* beta, float* out, int order) {
  for (int s = 0; s < T; s++)
    for (int t = 0; t < ntiles; t++) {
      long o = (long)s * step_stride + (long)t * dv;
      float tmp[256];
      orc_fp32_step_o(dk, dv, S + (long)t * dk * dv, q + o, k + o, v + o,
                      a + (long)s * a_step + (long)t * dk, beta[(long)s * ntiles + t],
                      out ? out + o : tmp, order);
    }
}

void orc_fp32_run(int dk, int dv, int ntiles, int T, float* S, const float* q, const float* k,
                  const float* v, long step_stride, const float* a, long a_step,
                  const float* beta, float* out) {
  orc_fp32_run_o(dk, dv, ntiles, T, S, q, k, v, step_stride, a, a_step, beta, out,
                 ORC_DELTA_FIRST);
}
