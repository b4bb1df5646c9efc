/*
 * iskv_oracle.c -- plain, slow fp64 CPU reference of the iS-KV compressed KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; it exists so that the tests, the smoke check and the CPU
 * baseline leg of the benchmark can check the GPU library against an
 * independent implementation. It shares no code, header, table or constant
 * with the HIP library.
 *
 * Source: page "iS-KV: Online Low-Rank KV Cache Compression via
 * Block-Incremental SVD".
 *   - Theory, objective and truncated SVD: section "Theoretical Foundation"
 *     (rank-constrained Frobenius objective; SVD_r keeps k = min(r, n, d)).
 *   - Window and history: section "Architecture Overview".
 *   - Update: section "Block-Incremental Decoding Updates" (residual
 *     E = F - (FB)B^T, residual basis P, core Z = [Sigma 0; FB FP],
 *     (G, Sigma+, H) = SVD_r(Z), U+ = [U 0; 0 I] G, B+ = [B P] H).
 *   - Reconstruction and storage: section "Reconstruction and Storage".
 *
 * Every routine is written as the definition or the algorithm step it
 * follows, with no blocking or reordering. Conventions:
 *   - matrices are row-major unless stated; d is the head dimension.
 *   - the history is stored as C = U Sigma (n x k), sigma (k) and the basis
 *     as Bt (k x d: row j is basis vector j). The coordinate update then
 *     needs no division by sigma: since Z H = G Sigma, C+ = [C 0; FB FP] H_r.
 *   - the core SVD is a textbook one-sided (Hestenes) Jacobi iteration with
 *     cyclic-by-rows ordering (Golub & Van Loan, "Matrix Computations",
 *     one-sided Jacobi; Demmel & Veselic 1992).
 *
 * Parity status: every exported function is pinned by the CPU tests against
 * closed forms, invariants, brute force or LAPACK (numpy); none is unpinned.
 * The ORA_PLANT_* switches (all off by default) plant one known mistake each;
 * a CPU test builds each variant and checks that the pins reject it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_OK 0
#define ORA_ERR_ARG -1
#define ORA_ERR_NOCONV -2
#define ORA_ERR_MEM -3

typedef struct {
  int k;            /* rank before the fold */
  int p;            /* residual basis size, min(b, d - k) */
  int kplus;        /* rank after the fold, min(r, k + p) */
  int sweeps;       /* Jacobi sweeps used */
  double discarded; /* sum of squared singular values dropped by truncation */
} ora_fold_info;

static double dot(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; i++) s += a[i] * b[i];
  return s;
}

/* ------------------------------------------------------------------------ */
/* One-sided Jacobi SVD of an m x c matrix.                                  */
/*   Z: column-major (column j at Z + j*m). On return its columns are        */
/*      mutually orthogonal: Z_out = Z_in * H.                               */
/*   H: c x c column-major, accumulated rotations (set to I here).           */
/*   sv: column norms of Z_out = singular values (unsorted).                 */
/* A pair (i, j) is rotated while |z_i.z_j| > m * 2^-53 * ||z_i|| ||z_j||.     */
/* Columns whose norm is at or below m * 2^-53 * ||Z||_F are at the rounding */
/* level of the matrix and are treated as zero (never rotated): otherwise a  */
/* core built from rows already inside span(B) would rotate its rounding     */
/* noise forever.                                                            */
/* Requires m >= c (more columns than rows can never be made orthogonal;     */
/* the fold's core always has k + b rows >= k + p columns).                  */
/* Returns the number of sweeps, or ORA_ERR_NOCONV after maxsweeps.          */
/* ------------------------------------------------------------------------ */
int ora_jacobi(int m, int c, double *Z, double *H, double *sv, int maxsweeps) {
  if (m < 0 || c < 0 || m < c) return ORA_ERR_ARG;
  const double tol = (double)(m > 1 ? m : 1) * ldexp(1.0, -53);
  double fro2 = 0.0;
  for (size_t t = 0; t < (size_t)m * c; t++) fro2 += Z[t] * Z[t];
  const double negligible = tol * tol * fro2;
  for (int j = 0; j < c; j++)
    for (int i = 0; i < c; i++) H[j * c + i] = (i == j) ? 1.0 : 0.0;
  int sweep = 0;
  int converged = (c < 2);
  while (!converged && sweep < maxsweeps) {
    sweep++;
    int rotations = 0;
    for (int i = 0; i < c - 1; i++) {
      for (int j = i + 1; j < c; j++) {
        double *zi = Z + (size_t)i * m, *zj = Z + (size_t)j * m;
        double alpha = dot(zi, zi, m);
        double beta = dot(zj, zj, m);
        double gamma = dot(zi, zj, m);
        if (alpha <= negligible || beta <= negligible) continue;
        if (!(fabs(gamma) > tol * sqrt(alpha * beta))) continue;
        /* rotation that zeroes the (i, j) entry of the 2x2 Gram matrix */
        double zeta = (beta - alpha) / (2.0 * gamma);
        double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        double cs = 1.0 / sqrt(1.0 + t * t);
        double sn = cs * t;
        for (int r = 0; r < m; r++) {
          double a = zi[r], b = zj[r];
#ifdef ORA_PLANT_ROT_SIGN
          zi[r] = cs * a + sn * b;
#else
          zi[r] = cs * a - sn * b;
#endif
          zj[r] = sn * a + cs * b;
        }
        double *hi = H + (size_t)i * c, *hj = H + (size_t)j * c;
        for (int r = 0; r < c; r++) {
          double a = hi[r], b = hj[r];
          hi[r] = cs * a - sn * b;
          hj[r] = sn * a + cs * b;
        }
        rotations++;
      }
    }
    if (rotations == 0) converged = 1;
  }
  for (int j = 0; j < c; j++) sv[j] = sqrt(dot(Z + (size_t)j * m, Z + (size_t)j * m, m));
  return converged ? sweep : ORA_ERR_NOCONV;
}

/* Singular values of an m x c row-major matrix X (sorted descending). */
int ora_singular_values(int m, int c, const double *X, double *sv_sorted, int maxsweeps) {
  double *Z = malloc(sizeof(double) * (size_t)m * c);
  double *H = malloc(sizeof(double) * (size_t)c * c);
  double *sv = malloc(sizeof(double) * (size_t)c);
  if (!Z || !H || !sv) { free(Z); free(H); free(sv); return ORA_ERR_MEM; }
  for (int i = 0; i < m; i++)
    for (int j = 0; j < c; j++) Z[(size_t)j * m + i] = X[(size_t)i * c + j];
  int rc = ora_jacobi(m, c, Z, H, sv, maxsweeps);
  /* selection sort, descending */
  for (int a = 0; a < c; a++) {
    int best = a;
    for (int b = a + 1; b < c; b++) if (sv[b] > sv[best]) best = b;
    double t = sv[a]; sv[a] = sv[best]; sv[best] = t;
    sv_sorted[a] = sv[a];
  }
  free(Z); free(H); free(sv);
  return rc;
}

/* Rank after a fold from rank k (section "Block-Incremental Decoding
 * Updates": p = min(b, d - k) residual directions, k+ = min(r, k + p)). */
static int kplus_after(int d, int b, int r, int k) {
  const int p = (b < d - k) ? b : d - k;
  return (r < k + p) ? r : k + p;
}

/* Orthogonalize v (length d) against the rows of `basis` (nb x d) by
 * modified Gram-Schmidt, two passes; returns the norm of the result. */
static double mgs2(double *v, const double *basis, int nb, int d) {
  for (int pass = 0; pass < 2; pass++)
    for (int q = 0; q < nb; q++) {
      const double *u = basis + (size_t)q * d;
      double c = dot(u, v, d);
      for (int t = 0; t < d; t++) v[t] -= c * u[t];
    }
  return sqrt(dot(v, v, d));
}

/* ------------------------------------------------------------------------ */
/* One block-incremental update (section "Block-Incremental Decoding         */
/* Updates").                                                                */
/*   d, b, r : head dim, block rows, rank budget                             */
/*   n, k    : history rows and current rank                                 */
/*   C       : history coordinates, row-major with leading dimension ldc     */
/*             (>= d); rows 0..n+b-1 must exist. Rows 0..n-1 hold U Sigma    */
/*             in columns 0..k-1. On return rows 0..n+b-1 hold U+ Sigma+.    */
/*   sigma   : length >= d; sigma[0..k-1] on entry, [0..kplus-1] on return   */
/*   Bt      : d x d row-major; rows 0..k-1 = basis vectors on entry         */
/*   F       : b x d pending block                                           */
/*   mode    : 0 = joint update of basis and coordinates (the method);       */
/*             1 = naive: basis updated, old rows keep their coordinates     */
/*             2 = fixed basis: once a basis exists (k > 0) it is kept;      */
/*                 new rows are stored as their projections F B, the rank,   */
/*                 sigma and the old rows stay, and `discarded` is the        */
/*                 residual energy ||F - F B B^T||^2 that is lost            */
/*   porder  : 0 = build P from the residual rows first to last, 1 = last    */
/*             to first (a different but equally valid residual basis)       */
/* ------------------------------------------------------------------------ */
int ora_fold(int d, int b, int r, int n, int k, double *C, int ldc, double *sigma,
             double *Bt, const double *F, int mode, int porder, ora_fold_info *info) {
  if (d <= 0 || b <= 0 || r <= 0 || r > d || k < 0 || k > d || k > r || n < 0 || ldc < d)
    return ORA_ERR_ARG;
  if (mode < 0 || mode > 2) return ORA_ERR_ARG;
  if (mode == 2 && k > 0) {
    /* Ablation "keeping bases fixed" ([iS-KV] Ablation Study): no residual
     * basis and no core SVD; the block is stored in the existing basis. */
    double lost = 0.0;
    for (int i = 0; i < b; i++) {
      const double *f = F + (size_t)i * d;
      double *ci = C + (size_t)(n + i) * ldc;
      double proj2 = 0.0;
      for (int j = 0; j < d; j++) {
        double y = (j < k) ? dot(f, Bt + (size_t)j * d, d) : 0.0;
        ci[j] = y;
        proj2 += y * y;
      }
      lost += dot(f, f, d) - proj2; /* B orthonormal: ||F - F B B^T||^2 */
    }
    if (info) {
      info->k = k;
      info->p = 0;
      info->kplus = k;
      info->sweeps = 0;
      info->discarded = lost;
    }
    return ORA_OK;
  }
  const int p = (b < d - k) ? b : d - k;
  const int m = k + b;  /* rows of Z */
  const int c = k + p;  /* columns of Z */
  const int kplus = (r < c) ? r : c;
  int rc = ORA_OK;

  double *Y = calloc((size_t)b * (k > 0 ? k : 1), sizeof(double));
  double *E = calloc((size_t)b * d, sizeof(double));
  double *Pt = calloc((size_t)(p > 0 ? p : 1) * d, sizeof(double));
  double *FP = calloc((size_t)b * (p > 0 ? p : 1), sizeof(double));
  double *Z = calloc((size_t)m * (c > 0 ? c : 1), sizeof(double));
  double *H = calloc((size_t)(c > 0 ? c : 1) * (c > 0 ? c : 1), sizeof(double));
  double *sv = calloc((size_t)(c > 0 ? c : 1), sizeof(double));
  int *perm = calloc((size_t)(c > 0 ? c : 1), sizeof(int));
  double *BP = calloc((size_t)(c > 0 ? c : 1) * d, sizeof(double));
  double *Bn = calloc((size_t)d * d, sizeof(double));
  double *sgn = calloc((size_t)(c > 0 ? c : 1), sizeof(double));
  double *tmp = calloc((size_t)d, sizeof(double));
  double *v = calloc((size_t)d, sizeof(double));
  if (!Y || !E || !Pt || !FP || !Z || !H || !sv || !perm || !BP || !Bn || !sgn || !tmp || !v) {
    rc = ORA_ERR_MEM;
    goto out;
  }

  /* Step 1: projection Y = F B and residual E = F - Y B^T, orthogonalized a
   * second time against B (E <- E - (E B) B^T). */
  for (int i = 0; i < b; i++)
    for (int j = 0; j < k; j++) Y[(size_t)i * k + j] = dot(F + (size_t)i * d, Bt + (size_t)j * d, d);
  for (int i = 0; i < b; i++) {
    double *e = E + (size_t)i * d;
    memcpy(e, F + (size_t)i * d, sizeof(double) * d);
    for (int j = 0; j < k; j++) {
      double y = Y[(size_t)i * k + j];
      for (int t = 0; t < d; t++) e[t] -= y * Bt[(size_t)j * d + t];
    }
    for (int j = 0; j < k; j++) {
      double y2 = dot(e, Bt + (size_t)j * d, d);
      for (int t = 0; t < d; t++) e[t] -= y2 * Bt[(size_t)j * d + t];
    }
  }

  /* Step 1 (cont.): residual basis P, p = min(b, d - k) orthonormal vectors,
   * orthogonal to B, spanning the residual rows. Modified Gram-Schmidt with
   * re-orthogonalization over the residual rows; if they span fewer than p
   * directions, completed with canonical vectors (skipping ones that lie in
   * the span already). BP = [B; P] as rows, so [B P] = BP^T. */
  for (int j = 0; j < k; j++) memcpy(BP + (size_t)j * d, Bt + (size_t)j * d, sizeof(double) * d);
  {
    double fnorm = 0.0;
    for (size_t t = 0; t < (size_t)b * d; t++) fnorm += F[t] * F[t];
    fnorm = sqrt(fnorm);
    int np = 0;
    for (int s = 0; s < b && np < p; s++) {
      int i = porder ? (b - 1 - s) : s;
      memcpy(v, E + (size_t)i * d, sizeof(double) * d);
      double nv = mgs2(v, BP, k + np, d);
      if (nv > 1e-12 * fnorm && nv > 0.0) {
#ifdef ORA_PLANT_P_UNNORMALIZED
        nv = 1.0;
#endif
        for (int t = 0; t < d; t++) BP[(size_t)(k + np) * d + t] = v[t] / nv;
        np++;
      }
    }
    for (int s = 0; s < d && np < p; s++) {
      int i = porder ? (d - 1 - s) : s;
      memset(v, 0, sizeof(double) * d);
      v[i] = 1.0;
      double nv = mgs2(v, BP, k + np, d);
      if (nv > 1e-3) {
        for (int t = 0; t < d; t++) BP[(size_t)(k + np) * d + t] = v[t] / nv;
        np++;
      }
    }
    if (np != p) { rc = ORA_ERR_ARG; goto out; }
    for (int j = 0; j < p; j++) memcpy(Pt + (size_t)j * d, BP + (size_t)(k + j) * d, sizeof(double) * d);
  }

  /* FP = F P (b x p). */
  for (int i = 0; i < b; i++)
    for (int j = 0; j < p; j++) FP[(size_t)i * p + j] = dot(F + (size_t)i * d, Pt + (size_t)j * d, d);

  /* Step 2: core Z = [Sigma 0; FB FP], (k+b) x (k+p), column-major. */
  for (int j = 0; j < k; j++) {
#ifdef ORA_PLANT_NO_SIGMA
    Z[(size_t)j * m + j] = 1.0;
#else
    Z[(size_t)j * m + j] = sigma[j];
#endif
#ifndef ORA_PLANT_DROP_FB
    for (int i = 0; i < b; i++) Z[(size_t)j * m + k + i] = Y[(size_t)i * k + j];
#endif
  }
  for (int j = 0; j < p; j++)
    for (int i = 0; i < b; i++) Z[(size_t)(k + j) * m + k + i] = FP[(size_t)i * p + j];

  /* Step 3: core SVD. After the iteration Z holds Z H = G Sigma+. */
  {
    int sw = ora_jacobi(m, c, Z, H, sv, 60);
    if (sw < 0) { rc = ORA_ERR_NOCONV; goto out; }
    if (info) info->sweeps = sw;
  }

  /* Order components by descending singular value (stable: ties keep the
   * lower column first); keep the leading kplus. */
  for (int j = 0; j < c; j++) perm[j] = j;
  for (int a = 1; a < c; a++) {
    int pj = perm[a];
    int q = a - 1;
#ifdef ORA_PLANT_SORT_ASC
    while (q >= 0 && sv[perm[q]] > sv[pj]) { perm[q + 1] = perm[q]; q--; }
#else
    while (q >= 0 && sv[perm[q]] < sv[pj]) { perm[q + 1] = perm[q]; q--; }
#endif
    perm[q + 1] = pj;
  }

  /* B+ = [B P] H_r, with each column's sign fixed so that its entry of
   * largest magnitude (lowest index on ties) is positive. */
  for (int jj = 0; jj < kplus; jj++) {
    const double *h = H + (size_t)perm[jj] * c;
    for (int t = 0; t < d; t++) {
      double s = 0.0;
      for (int i = 0; i < c; i++) s += BP[(size_t)i * d + t] * h[i];
      Bn[(size_t)jj * d + t] = s;
    }
    int am = 0;
    for (int t = 1; t < d; t++)
      if (fabs(Bn[(size_t)jj * d + t]) > fabs(Bn[(size_t)jj * d + am])) am = t;
    sgn[jj] = (Bn[(size_t)jj * d + am] < 0.0) ? -1.0 : 1.0;
    for (int t = 0; t < d; t++) Bn[(size_t)jj * d + t] *= sgn[jj];
  }

  /* U+ Sigma+ = [U 0; 0 I] G Sigma+ = [C 0; FB FP] H_r.
   * Old rows: C[i] <- C[i] H[0:k, r-cols] (joint), or kept (naive).
   * New rows: bottom b rows of the rotated core, (Z H)[k + i]. */
  for (int i = 0; i < n; i++) {
    double *ci = C + (size_t)i * ldc;
#ifdef ORA_PLANT_NO_REWRITE
    if (0) {
#else
    if (mode == 0) {
#endif
      for (int jj = 0; jj < kplus; jj++) {
        const double *h = H + (size_t)perm[jj] * c;
        double s = 0.0;
#ifdef ORA_PLANT_H_TRANSPOSE
        for (int l = 0; l < k; l++) s += ci[l] * H[(size_t)l * c + perm[jj]];
#else
        for (int l = 0; l < k; l++) s += ci[l] * h[l];
#endif
        tmp[jj] = sgn[jj] * s;
      }
      for (int jj = 0; jj < d; jj++) ci[jj] = (jj < kplus) ? tmp[jj] : 0.0;
    } else {
#if defined(ORA_PLANT_NAIVE_SIGN)
      for (int jj = 0; jj < kplus; jj++) ci[jj] *= sgn[jj];
#elif defined(ORA_PLANT_NAIVE_PERM)
      for (int jj = 0; jj < kplus; jj++) tmp[jj] = (perm[jj] < k) ? ci[perm[jj]] : 0.0;
      for (int jj = 0; jj < kplus; jj++) ci[jj] = tmp[jj];
#endif
      for (int jj = kplus; jj < d; jj++) ci[jj] = 0.0;
    }
  }
  for (int i = 0; i < b; i++) {
    double *ci = C + (size_t)(n + i) * ldc;
    for (int jj = 0; jj < d; jj++)
#ifdef ORA_PLANT_NEWROW_OFFSET
      ci[jj] = (jj < kplus) ? sgn[jj] * Z[(size_t)perm[jj] * m + i] : 0.0;
#else
      ci[jj] = (jj < kplus) ? sgn[jj] * Z[(size_t)perm[jj] * m + k + i] : 0.0;
#endif
  }

  /* Commit sigma+, B+ and the discarded energy. */
  {
    double disc = 0.0;
#ifdef ORA_PLANT_DISCARD_UNSQUARED
    for (int jj = kplus; jj < c; jj++) disc += sv[perm[jj]];
#else
    for (int jj = kplus; jj < c; jj++) disc += sv[perm[jj]] * sv[perm[jj]];
#endif
    for (int jj = 0; jj < d; jj++) sigma[jj] = (jj < kplus) ? sv[perm[jj]] : 0.0;
    for (int jj = 0; jj < d; jj++)
      for (int t = 0; t < d; t++) Bt[(size_t)jj * d + t] = (jj < kplus) ? Bn[(size_t)jj * d + t] : 0.0;
    if (info) {
      info->k = k;
      info->p = p;
      info->kplus = kplus;
      info->discarded = disc;
    }
  }

out:
  free(Y); free(E); free(Pt); free(FP); free(Z); free(H); free(sv); free(perm);
  free(BP); free(Bn); free(sgn); free(tmp); free(v);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Low-bit storage of the history coordinates. The page's "Conclusion" names  */
/* integration with quantization as the way to cut memory further, and the   */
/* JoLT abstract on the "Tensor Decomposition of Transformer Key-Value        */
/* Caches" page keeps its factors in low precision; neither fixes a format.   */
/* Reading taken here: symmetric int8 codes with one scale per stored row.    */
/* For row c (columns 0..k-1) with m = max_j |c_j|:                           */
/*   scale s = m / 127,  code q_j = round-half-even(127 c_j / m)              */
/* (a zero row has s = 0 and q = 0); the stored value is q_j s, so the row's  */
/* largest entry keeps its magnitude and every entry moves by at most s / 2.  */
/* In place: rows 0..rows-1 of C (leading dimension ldc) become their stored  */
/* values; columns k.. are set to zero. Q (rows x ldq) and scale (rows)       */
/* receive the codes and scales when they are not NULL.                       */
/* ------------------------------------------------------------------------ */
void ora_store_i8(int rows, int k, int ldc, double *C, int8_t *Q, int ldq, double *scale) {
  for (int i = 0; i < rows; i++) {
    double *c = C + (size_t)i * ldc;
    double m = 0.0;
    for (int j = 0; j < k; j++) m = fabs(c[j]) > m ? fabs(c[j]) : m;
#ifdef ORA_PLANT_Q8_SCALE128
    const double levels = 128.0;
#else
    const double levels = 127.0;
#endif
    const double s = m / levels;
    for (int j = 0; j < ldc; j++) {
      double q = 0.0;
      if (j < k && m > 0.0) {
        const double x = levels * c[j] / m;
#if defined(ORA_PLANT_Q8_TRUNC)
        q = trunc(x);
#elif defined(ORA_PLANT_Q8_HALFAWAY)
        q = round(x);
#else
        q = nearbyint(x); /* default rounding mode: to nearest, ties to even */
#endif
      }
      if (Q && j < ldq) Q[(size_t)i * ldq + j] = (int8_t)q;
      c[j] = q * s;
    }
    if (scale) scale[i] = s;
  }
}

/* int8 storage of a history (rows 0..rows-1 of C = U Sigma, k columns):    */
/* the stored factor is U = C Sigma^-1, the one the page's equation for U+    */
/* updates, whose rows have comparable entries (a row of U Sigma inherits the */
/* power-law decay of sigma, so one scale per row would waste the codes of   */
/* its small coordinates). Each row of U is stored by ora_store_i8 and C      */
/* becomes U_stored Sigma. Columns with sigma_j = 0 are zero. Q and scale as  */
/* in ora_store_i8 (codes and scales of U).                                  */
void ora_store_u_i8(int rows, int k, int ldc, double *C, const double *sigma, int8_t *Q, int ldq,
                    double *scale) {
  for (int i = 0; i < rows; i++) {
    double *c = C + (size_t)i * ldc;
    for (int j = 0; j < k; j++)
#ifdef ORA_PLANT_Q8_STORE_C
      (void)sigma;
#else
      c[j] = sigma[j] > 0.0 ? c[j] / sigma[j] : 0.0;
#endif
    ora_store_i8(1, k, ldc, c, Q ? Q + (size_t)i * ldq : NULL, ldq, scale ? scale + i : NULL);
#ifndef ORA_PLANT_Q8_STORE_C
    for (int j = 0; j < k; j++) c[j] *= sigma[j];
#endif
  }
}

/* One update with int8 coordinate storage: the fold of the method on the     */
/* stored history, then every stored row is stored again (ora_store_u_i8      */
/* with the new sigma): the n old rows after their rotation and the b new     */
/* rows. Sigma and the basis are the fold's. Rows 0..n-1 of C must hold       */
/* stored values.                                                            */
int ora_fold_i8(int d, int b, int r, int n, int k, double *C, int ldc, double *sigma, double *Bt,
                const double *F, int porder, ora_fold_info *info) {
  int rc = ora_fold(d, b, r, n, k, C, ldc, sigma, Bt, F, 0, porder, info);
  if (rc) return rc;
  const int kplus = info ? info->kplus : kplus_after(d, b, r, k);
#ifdef ORA_PLANT_Q8_OLDROWS
  ora_store_u_i8(b, kplus, ldc, C + (size_t)n * ldc, sigma, NULL, 0, NULL);
#else
  ora_store_u_i8(n + b, kplus, ldc, C, sigma, NULL, 0, NULL);
#endif
  return ORA_OK;
}

/* ------------------------------------------------------------------------ */
/* One-shot prefill (section "Prefill Compression": the prompt's rows are    */
/* factorised at once by a truncated SVD; key and value protection are not  */
/* modelled, so every row goes to the history).                              */
/*   X     : N x d prompt rows, row-major                                    */
/*   C     : N x ldc (ldc >= d); on return rows hold U_r Sigma_r in columns  */
/*           0..kplus-1, zeros beyond                                        */
/*   sigma : d; Bt : d x d (rows 0..kplus-1 = right singular vectors, each   */
/*           signed so that its entry of largest magnitude is positive)      */
/* kplus = min(r, N, d) (section "Theoretical Foundation": SVD_r keeps       */
/* k = min(r, n, d)). The SVD is the same one-sided Jacobi as the fold's     */
/* core, applied to X itself (padded with zero rows to d rows when N < d,    */
/* which changes neither the singular values nor the right vectors).         */
/* info (optional): k = 0, p = N, kplus, sweeps, discarded energy.           */
/* Returns kplus, or a negative error.                                       */
/* ------------------------------------------------------------------------ */
int ora_prefill_oneshot(int d, int r, int N, const double *X, double *C, int ldc, double *sigma,
                        double *Bt, ora_fold_info *info) {
  if (d <= 0 || r <= 0 || N <= 0 || ldc < d) return ORA_ERR_ARG;
  const int m = N > d ? N : d;
  const int kplus = (r < N ? r : N) < d ? (r < N ? r : N) : d;
  int rc = 0;
  double *Z = calloc((size_t)m * d, sizeof(double));
  double *H = calloc((size_t)d * d, sizeof(double));
  double *sv = calloc((size_t)d, sizeof(double));
  int *perm = calloc((size_t)d, sizeof(int));
  double *sgn = calloc((size_t)d, sizeof(double));
  if (!Z || !H || !sv || !perm || !sgn) { rc = ORA_ERR_MEM; goto out; }
  /* Z = X column-major (column t holds feature t of every row) */
  for (int i = 0; i < N; i++)
    for (int t = 0; t < d; t++) Z[(size_t)t * m + i] = X[(size_t)i * d + t];
  {
    int sw = ora_jacobi(m, d, Z, H, sv, 60);
    if (sw < 0) { rc = ORA_ERR_NOCONV; goto out; }
    if (info) info->sweeps = sw;
  }
  for (int j = 0; j < d; j++) perm[j] = j;
  for (int a = 1; a < d; a++) {
    int pj = perm[a];
    int q = a - 1;
    while (q >= 0 && sv[perm[q]] < sv[pj]) { perm[q + 1] = perm[q]; q--; }
    perm[q + 1] = pj;
  }
  /* basis vector jj = column perm[jj] of H = V, signed by its largest entry */
  for (int jj = 0; jj < d; jj++) {
    const double *h = H + (size_t)perm[jj] * d;
    int am = 0;
    for (int t = 1; t < d; t++)
      if (fabs(h[t]) > fabs(h[am])) am = t;
    sgn[jj] = (h[am] < 0.0) ? -1.0 : 1.0;
    for (int t = 0; t < d; t++) Bt[(size_t)jj * d + t] = (jj < kplus) ? sgn[jj] * h[t] : 0.0;
  }
  /* U_r Sigma_r = X V_r: the rotated columns (X H) of the kept components */
  for (int i = 0; i < N; i++)
    for (int jj = 0; jj < ldc; jj++)
      C[(size_t)i * ldc + jj] = (jj < kplus) ? sgn[jj] * Z[(size_t)perm[jj] * m + i] : 0.0;
  {
    double disc = 0.0;
    for (int jj = kplus; jj < d; jj++) disc += sv[perm[jj]] * sv[perm[jj]];
    for (int jj = 0; jj < d; jj++) sigma[jj] = (jj < kplus) ? sv[perm[jj]] : 0.0;
    if (info) {
      info->k = 0;
      info->p = N;
      info->kplus = kplus;
      info->discarded = disc;
    }
  }
  rc = kplus;
out:
  free(Z); free(H); free(sv); free(perm); free(sgn);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Whole stream of one unit (section "Architecture Overview": exact recent   */
/* window of w rows plus low-rank history).                                  */
/*   X        : N x d rows in arrival order                                  */
/*   prefill  : the first `prefill` rows (a multiple of b) fold directly     */
/*   Then rows arrive one at a time; when the window holds >= w + b rows,    */
/*   its oldest b rows fold into the history.                                */
/* Outputs (caller-allocated):                                               */
/*   C (N x d, ldc = d), sigma (d), Bt (d x d), win_first (index into X of   */
/*   the oldest window row), and counts[3] = {n, e, k}.                      */
/*   log (optional, 5 doubles per fold): k, p, kplus, sweeps, discarded.     */
/*   store    : 0 = fp64 coordinates; 1 = int8 rows with per-row scales      */
/*              (ora_fold_i8; joint mode only), C then holds stored values.  */
/* Returns the number of folds, or a negative error.                         */
/* ------------------------------------------------------------------------ */
int ora_run(int d, int b, int r, int w, int N, int prefill, const double *X, int mode,
            int store, double *C, double *sigma, double *Bt, int *counts, double *log, int log_cap) {
  if (prefill < 0 || prefill % b != 0 || prefill > N) return ORA_ERR_ARG;
  if (store < 0 || store > 1 || (store == 1 && mode != 0)) return ORA_ERR_ARG;
  int n = 0, k = 0, folds = 0;
  memset(sigma, 0, sizeof(double) * d);
  memset(Bt, 0, sizeof(double) * d * d);
  int first = 0;  /* index of the oldest unfolded row */
  ora_fold_info info;
  for (int s = 0; s < prefill; s += b) {
#if defined(ORA_PLANT_PREFILL_REVERSED)
    const double *Fs = X + (size_t)(prefill - b - s) * d;
#else
    const double *Fs = X + (size_t)s * d;
#endif
#if defined(ORA_PLANT_PREFILL_JOINT)
    int rc = ora_fold(d, b, r, n, k, C, d, sigma, Bt, Fs, 0, 0, &info);
#else
    int rc = store ? ora_fold_i8(d, b, r, n, k, C, d, sigma, Bt, Fs, 0, &info)
                   : ora_fold(d, b, r, n, k, C, d, sigma, Bt, Fs, mode, 0, &info);
#endif
    if (rc) return rc;
    if (log && folds < log_cap) {
      double *lg = log + (size_t)folds * 5;
      lg[0] = info.k; lg[1] = info.p; lg[2] = info.kplus; lg[3] = info.sweeps; lg[4] = info.discarded;
    }
    folds++;
    n += b;
    k = info.kplus;
  }
  first = prefill;
  for (int t = prefill; t < N; t++) {
    int e = t + 1 - first;
    if (e >= w + b) {
      const double *Fw = X + (size_t)first * d;
      int rc = store ? ora_fold_i8(d, b, r, n, k, C, d, sigma, Bt, Fw, 0, &info)
                     : ora_fold(d, b, r, n, k, C, d, sigma, Bt, Fw, mode, 0, &info);
      if (rc) return rc;
      if (log && folds < log_cap) {
        double *lg = log + (size_t)folds * 5;
        lg[0] = info.k; lg[1] = info.p; lg[2] = info.kplus; lg[3] = info.sweeps; lg[4] = info.discarded;
      }
      folds++;
      n += b;
      k = info.kplus;
      first += b;
    }
  }
  counts[0] = n;
  counts[1] = N - first;
  counts[2] = k;
  return folds;
}

/* Reconstruction (section "Reconstruction and Storage"): history rows
 * (U Sigma B^T)[j] = C[j] B^T followed by the exact window rows.
 * C: n x ldc, Bt: k x d, W: e x d; out: (n + e) x d. */
void ora_reconstruct(int d, int n, int k, int ldc, const double *C, const double *Bt, int e,
                     const double *W, double *out) {
  for (int i = 0; i < n; i++)
    for (int t = 0; t < d; t++) {
      double s = 0.0;
#ifdef ORA_PLANT_RECON_WRONG_ROW
      for (int j = 0; j < k; j++) s += C[(size_t)i * ldc + j] * Bt[(size_t)j * d + (d - 1 - t)];
#else
      for (int j = 0; j < k; j++) s += C[(size_t)i * ldc + j] * Bt[(size_t)j * d + t];
#endif
      out[(size_t)i * d + t] = s;
    }
  memcpy(out + (size_t)n * d, W, sizeof(double) * (size_t)e * d);
}

/* Dense single-query attention over reconstructed rows, for g query heads
 * sharing one KV head: out_h = softmax(scale * Kt q_h)^T Vt.
 * Kt, Vt: T x d; q, out: g x d. */
void ora_attend(int d, int T, int g, const double *Kt, const double *Vt, const double *q,
                double scale, double *out) {
  double *s = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  for (int h = 0; h < g; h++) {
    const double *qh = q + (size_t)h * d;
    double mx = -INFINITY;
    for (int i = 0; i < T; i++) {
#ifdef ORA_PLANT_ATTEND_NOSCALE
      s[i] = dot(Kt + (size_t)i * d, qh, d);
#else
      s[i] = scale * dot(Kt + (size_t)i * d, qh, d);
#endif
      if (s[i] > mx) mx = s[i];
    }
    double den = 0.0;
    for (int i = 0; i < T; i++) { s[i] = exp(s[i] - mx); den += s[i]; }
    for (int t = 0; t < d; t++) {
      double acc = 0.0;
      for (int i = 0; i < T; i++) acc += s[i] * Vt[(size_t)i * d + t];
      out[(size_t)h * d + t] = (T > 0) ? acc / den : 0.0;
    }
  }
  free(s);
}

/* Per-layer persistent storage in bytes (section "Reconstruction and
 * Storage"): beta_f * sum_X k_X (n_X + d + 1) + beta_e * d * sum_X e_X. */
double ora_storage_bytes(int d, int kk, int nk, int ek, int kv, int nv, int ev, double beta_f,
                         double beta_e) {
#ifdef ORA_PLANT_STORAGE_NO_SIGMA
  return beta_f * ((double)kk * (nk + d) + (double)kv * (nv + d)) +
#else
  return beta_f * ((double)kk * (nk + d + 1) + (double)kv * (nv + d + 1)) +
#endif
         beta_e * d * ((double)ek + ev);
}
