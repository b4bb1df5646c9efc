// Fold core of the joint update: one 512-thread workgroup per unit stream.
//
// Page "iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental
// SVD", section "Block-Incremental Decoding Updates":
//   1. residual E = F - (F B) B^T (orthogonalized twice against B) and a
//      residual basis P: the Householder QR of the d x (k+b) matrix
//      [B | E^T]; P = Q[:, k:k+p], p = min(b, d-k), and F P is read off the
//      triangular factor (F P = R[k:k+p, k:k+b]^T).
//   2. core Z = [Sigma 0; FB FP], (k+b) x (k+p).
//   3. (G, Sigma+, H) = SVD_r(Z), then B+ = [B P] H_r, and the coordinates
//      C+ = [C 0; FB FP] H_r (U+ Sigma+ without a division by sigma, since
//      Z H = G Sigma): this kernel writes the b new rows and H_top = H[0:k, :k+];
//      k_rewrite.hip streams the n old rows through H_top.
//
// The SVD of Z goes through its triangular factor: Z = Q_Z R (one structured
// Householder step, since the top k rows of Z are diagonal), and a one-sided
// Jacobi on the columns of R^T (the rows of R) converges to R^T W = H Sigma,
// so the right singular vectors are the converged columns over their norms
// and no rotation has to be accumulated (half the work of rotating columns
// of Z and of H together). A kept column at the rounding level (Z of lower
// rank than k+) is completed to an orthonormal H by Gram-Schmidt on unit
// vectors. The sort, sign rule, re-orthonormalisation and coordinate
// formulas are those of the fixed-coordinate core (k_core.hip).
//
// Work mapping: quads (4 lanes) own one column in the two QRs and of P;
// octets (8 lanes) own one Jacobi pair, 64 pairs per round, so a 128-column
// core keeps all 8 waves busy with 16 rows per lane.
#include "fold_common.hpp"

namespace iskv {

namespace {

using namespace fold;

constexpr int NTF = 512;  // threads per workgroup (8 wavefronts)
constexpr int LPJ = 8;    // lanes per Jacobi pair

// Jacobi column layout: c columns of length c (the rows of R), lane o of an
// octet holds rows o * 4 NQ .. + 4 NQ - 1, NQ = ceil(c / 32)
__host__ __device__ inline int fold_nq(int c) { return (c + 31) / 32; }
__host__ __device__ inline int fold_sj(int c) { return 8 * 4 * fold_nq(c) + 4; }

struct FoldLds {
  int big, small, total;  // floats: phase region, small arrays (offset = big), total
};

// small arrays: tau[D] sv[D] sgn[D] perm[D] nrm[D doubles] part[NTF] (part is also the
// reflector buffer of the QR of Z: 2 x 4 RB <= 256 floats)
constexpr int SMALL_FLOATS = 6 * D + NTF;

__host__ __device__ inline FoldLds fold_lds(int k, int b, int r) {
  FoldLds L;
  const int p = (b < D - k) ? b : D - k;
  const int m = k + b, c = k + p;
  const int kp = (r < c) ? r : c;
  const int sj = fold_sj(c);
  const int a = m * LDA;                   // [B | E^T] as rows
  const int h = c * sj;                    // R^T / H
  const int bp = kp * (D > sj ? D : sj);  // B+ staging, then H_r G
  int big = a;
  if (h + bp > big) big = h + bp;
  L.big = (big + 3) / 4 * 4;
  L.small = SMALL_FLOATS;
  L.total = L.big + L.small;
  return L;
}

template <int NQ>
__device__ __forceinline__ void run_jacobi(float *J, double *nrm, int sj, int c, double tol, double negl,
                                           int &sweep, bool &conv) {
  jacobi_columns<NTF, LPJ, NQ>(J, nrm, sj, c, tol, negl, sweep, conv);
}

// sum of a[e] * b[e] over N entries in four independent accumulation chains
// (a dependent chain of N fmas is latency-bound)
template <int N>
__device__ __forceinline__ float dot_chains(const float *a, const float *b) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < N; e++) p[e & 3] = fmaf(a[e], b[e], p[e & 3]);
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// Householder QR (LAPACK dlarfg convention: H = I - tau v v^T, v = 1 on row
// j, H x = beta e_j) of ncol <= NTF / 4 columns of length D held in registers:
// quad qid owns column qid, lane q rows 32q .. 32q + 31 (x). nref reflectors.
// The owner of column j builds reflector j, stores v (zeros above row j, 1 on
// it) in LDS row j of V (stride LDA; the rows must be free) and tau[j]; the
// other quads apply it from LDS. The owner of column j + 1 builds reflector
// j + 1 right after applying reflector j: one barrier per reflector. On
// return quad col holds column col of R (zero below the diagonal for col <
// nref) and V / tau define Q = H_0 ... H_{nref-1}.
__device__ __forceinline__ void qr_columns_in_registers(float *V, float (&x)[D / 4], int ncol, int nref,
                                                        float *tau) {
  const int tid = threadIdx.x, q = tid & 3, qid = tid >> 2;
  auto build = [&](int j) {
    float xm[D / 4], x0 = 0.f;
#pragma unroll
    for (int e = 0; e < D / 4; e++) {
      const int row = 32 * q + e;
      xm[e] = (row > j) ? x[e] : 0.f;
      x0 += (row == j) ? x[e] : 0.f;
    }
    const float s = quad_sum(dot_chains<D / 4>(xm, xm));
    x0 = quad_sum(x0);
    float tj = 0.f, beta = x0, scal = 0.f;
    if (s != 0.f) {  // a non-finite column reaches R (and is flagged later) instead of being skipped
      beta = -copysignf(sqrtf(x0 * x0 + s), x0);
      tj = (beta - x0) / beta;
      scal = 1.f / (x0 - beta);
    }
    float4 *vj = (float4 *)(V + (size_t)j * LDA + 32 * q);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float t[4];
#pragma unroll
      for (int z = 0; z < 4; z++) {
        const int row = 32 * q + 4 * e + z;
        t[z] = (row > j) ? x[4 * e + z] * scal : ((row == j) ? 1.f : 0.f);
      }
      vj[e] = float4{t[0], t[1], t[2], t[3]};
    }
#pragma unroll
    for (int e = 0; e < D / 4; e++) {
      const int row = 32 * q + e;
      x[e] = (row == j) ? beta : ((row > j) ? 0.f : x[e]);
    }
    if (q == 0) tau[j] = tj;
  };
  if (nref > 0 && qid == 0) build(0);
  __syncthreads();
  for (int j = 0; j < nref; j++) {
    const float tj = tau[j];
    if (tj != 0.f && qid > j && qid < ncol) {
      const float4 *vj = (const float4 *)(V + (size_t)j * LDA + 32 * q);
      float v[D / 4];
      float w = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float4 t = vj[e];
        v[4 * e] = t.x;
        v[4 * e + 1] = t.y;
        v[4 * e + 2] = t.z;
        v[4 * e + 3] = t.w;
      }
      w = tj * quad_sum(dot_chains<D / 4>(v, x));
#pragma unroll
      for (int e = 0; e < D / 4; e++) x[e] -= w * v[e];
    }
    if (j + 1 < nref && qid == j + 1) build(j + 1);
    __syncthreads();
  }
}

// R of Z = [diag(sigma) 0; Y] where Y (b x c) holds the block rows [F B | F P]:
// one structured Householder step per column. Reflector j (LAPACK dlarfg
// convention, H = I - tau v v^T with v = 1 on row j of R) touches only row j
// of R and the b block rows, since the rows of R below its diagonal are zero
// and stay zero. R is written as R^T in the Jacobi layout (column j of J =
// row j of R, J[j sj + j] = sigma_j on entry for j < k, zero elsewhere). The
// block column col lives in the registers of quad col (lane q: rows
// q RB .. q RB + RB - 1); the owner of column j + 1 builds reflector j + 1 as
// soon as it has applied reflector j and publishes its block part in vbuf
// (two buffers of 4 RB floats, alternating), so there is one barrier per
// reflector.
template <int RB>
__device__ __forceinline__ void tsqr_core(float *J, int sj, int c, int b, const float *Y, float *vbuf,
                                          float *tau) {
  const int tid = threadIdx.x, q = tid & 3, col = tid >> 2;
  float x[RB];
#pragma unroll
  for (int e = 0; e < RB; e++) {
    const int row = q * RB + e;
    x[e] = (col < c && row < b) ? Y[(size_t)row * D + col] : 0.f;
  }
  auto build = [&](int j) {  // quad j: reflector j from R[j][j] and its block column
    const float s = quad_sum(dot_chains<RB>(x, x));
    const float x0 = J[(size_t)j * sj + j];
    float tj = 0.f, beta = x0, scal = 0.f;
    if (s != 0.f) {  // a non-finite block reaches R (and is flagged later) instead of being skipped
      beta = -copysignf(sqrtf(x0 * x0 + s), x0);
      tj = (beta - x0) / beta;
      scal = 1.f / (x0 - beta);
    }
    float4 *vb = (float4 *)(vbuf + (j & 1) * 4 * RB + q * RB);
#pragma unroll
    for (int e = 0; e < RB / 4; e++)
      vb[e] = float4{x[4 * e] * scal, x[4 * e + 1] * scal, x[4 * e + 2] * scal, x[4 * e + 3] * scal};
    if (q == 0) {
      J[(size_t)j * sj + j] = beta;
      tau[j] = tj;
    }
#pragma unroll
    for (int e = 0; e < RB; e++) x[e] = 0.f;  // the block part of column j is annihilated
  };
  if (col == 0) build(0);
  __syncthreads();
  for (int j = 0; j < c; j++) {
    const float tj = tau[j];
    if (tj != 0.f && col > j && col < c) {
      const float4 *vb = (const float4 *)(vbuf + (j & 1) * 4 * RB + q * RB);
      float v[RB];
      float w = 0.f;
#pragma unroll
      for (int e = 0; e < RB / 4; e++) {
        const float4 t = vb[e];
        v[4 * e] = t.x;
        v[4 * e + 1] = t.y;
        v[4 * e + 2] = t.z;
        v[4 * e + 3] = t.w;
      }
      const float rjc = J[(size_t)j * sj + col];
      w = tj * (rjc + quad_sum(dot_chains<RB>(v, x)));
#pragma unroll
      for (int e = 0; e < RB; e++) x[e] -= w * v[e];
      if (q == 0) J[(size_t)j * sj + col] = rjc - w;
    }
    if (j + 1 < c && col == j + 1) build(j + 1);
    __syncthreads();
  }
}

// XK (0 keys, 1 values) is a template constant so that every access to the
// kernel arguments has a constant offset.
template <int NR, typename TK, typename TC, int XK>
__device__ __forceinline__ void fold_body(const FoldArgs &a, float *smem) {
  const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4;
  const int q = tid & 3, qid = tid >> 2;
  const int u = a.u0 + blockIdx.x;
  const Stream &X = a.X[XK];
  const int b = a.b, k = a.k[XK], r = a.r[XK];
  const int p = (b < D - k) ? b : D - k;
  const int c = k + p;
  const int kplus = (r < c) ? r : c;
  const int sj = fold_sj(c);
  const FoldLds lay = fold_lds(k, b, r);

  float *tau = smem + lay.big;
  float *sv = tau + D;
  float *sgn = sv + D;
  int *perm = (int *)(sgn + D);
  double *nrm = (double *)(perm + D);
  float *part = (float *)(nrm + D);

  const float *Bt = X.Bt + (size_t)u * r * D;
  float *Pg = X.P + (size_t)u * a.pmax * D;
  float *YFP = X.YFP + (size_t)u * a.bmax * D;
  const TK *ring = (const TK *)X.ring + (size_t)u * a.rcap * D;
  const float *sig_old = X.sig + (size_t)u * r;

  // ---------------- phase A: projection, residual, residual basis ---------
  float *A = smem;  // rows 0..k-1 = basis vectors, rows k..k+b-1 = residual rows (stride LDA)
  for (int i0 = tid; i0 < k * (D / 4); i0 += 4 * NTF) {
    float4 bq[4];
#pragma unroll
    for (int z = 0; z < 4; z++) {
      const int idx = i0 + NTF * z;
      if (idx < k * (D / 4)) bq[z] = reinterpret_cast<const float4 *>(Bt)[idx];
    }
#pragma unroll
    for (int z = 0; z < 4; z++) {
      const int idx = i0 + NTF * z;
      if (idx < k * (D / 4)) {
        const int row = idx / (D / 4), c4 = idx - row * (D / 4);
        *reinterpret_cast<float4 *>(A + (size_t)row * LDA + 4 * c4) = bq[z];
      }
    }
  }
  constexpr int NGR = NTF / 16;  // 16-lane row groups
  float f[NR][8];
#pragma unroll
  for (int qq = 0; qq < NR; qq++) {
    const int i = grp + NGR * qq;
    if (i < b) {
      int ri = a.head + i;
      if (ri >= a.rcap) ri -= a.rcap;
#pragma unroll
      for (int t = 0; t < 8; t++) f[qq][t] = ldf<TK>(ring, (size_t)ri * D + lane * 8 + t);
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++) f[qq][t] = 0.f;
    }
  }
  __syncthreads();
  // When k + b >= d the residual basis has p = d - k columns: it is any
  // orthonormal basis of the complement of B (the residual rows lie in it),
  // so it comes from the QR of B alone and E is not needed.
  const bool cmpl = (k + b >= D);
  const int nref = cmpl ? k : c;  // reflectors that define P
  // Y = F B and E = F - Y B^T; then once more E <- E - (E B) B^T
  for (int pass = 0; pass < (cmpl ? 1 : 2); pass++) {
    for (int j = 0; j < k; j++) {
      float bj[8];
#pragma unroll
      for (int t = 0; t < 8; t++) bj[t] = A[j * LDA + lane * 8 + t];
#pragma unroll
      for (int qq = 0; qq < NR; qq++) {
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < 8; t++) s += f[qq][t] * bj[t];
        s = sum16(s);
        if (!cmpl) {
#pragma unroll
          for (int t = 0; t < 8; t++) f[qq][t] -= s * bj[t];
        }
        const int i = grp + NGR * qq;
        if (pass == 0 && lane == 0 && i < b) YFP[i * D + j] = s;
      }
    }
  }
  if (!cmpl) {
#pragma unroll
    for (int qq = 0; qq < NR; qq++) {
      const int i = grp + NGR * qq;
      if (i < b) {
#pragma unroll
        for (int t = 0; t < 8; t++) A[(k + i) * LDA + lane * 8 + t] = f[qq][t];
      }
    }
  }
  __syncthreads();

  if (p > 0) {
    // Householder QR of [B | E^T] (column j = LDS row j), c reflectors; of B
    // alone (k reflectors) when P is the complement of B. Each column lives in
    // the registers of one quad (lane q: rows 32q .. 32q + 31); reflector j
    // (v = 1 on row j, zero above) is stored in LDS row j once the columns are
    // loaded.
    const int ncol = cmpl ? k : k + b;  // <= 127 columns: one quad each
    float x[D / 4];
    if (qid < ncol) {
      const float4 *src = (const float4 *)(A + (size_t)qid * LDA + 32 * q);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float4 t = src[e];
        x[4 * e] = t.x;
        x[4 * e + 1] = t.y;
        x[4 * e + 2] = t.z;
        x[4 * e + 3] = t.w;
      }
    }
    __syncthreads();  // LDS rows are free for the reflectors
    qr_columns_in_registers(A, x, ncol, nref, tau);
    if (!cmpl && qid >= k && qid < ncol) {
      // F P = R[k:k+p, k:k+b]^T (lower trapezoidal): column k + i of R gives row i
      const int i = qid - k;
#pragma unroll
      for (int e = 0; e < D / 4; e++) {
        const int row = 32 * q + e;
        if (row >= k && row < k + p) YFP[(size_t)i * D + row] = (row - k <= i) ? x[e] : 0.f;
      }
    }
    // P = Q[:, k:k+p] = H_0 ... H_{nref-1} [e_k .. e_{k+p-1}], accumulated
    // backwards in the registers of one quad per column; reflectors j > k+col
    // leave e_{k+col} unchanged and are skipped.
    for (int col = qid; col < p; col += NTF / 4) {
#pragma unroll
      for (int e = 0; e < D / 4; e++) x[e] = (32 * q + e == k + col) ? 1.f : 0.f;
      for (int j = min(k + col, nref - 1); j >= 0; j--) {
        const float tj = tau[j];
        if (tj == 0.f) continue;
        const float4 *vj = (const float4 *)(A + (size_t)j * LDA + 32 * q);
        float v[D / 4];
        float w = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float4 t = vj[e];
          v[4 * e] = t.x;
          v[4 * e + 1] = t.y;
          v[4 * e + 2] = t.z;
          v[4 * e + 3] = t.w;
        }
        w = tj * quad_sum(dot_chains<D / 4>(v, x));
#pragma unroll
        for (int e = 0; e < D / 4; e++) x[e] -= w * v[e];
      }
      float4 *dst = (float4 *)(Pg + (size_t)col * D + 32 * q);
#pragma unroll
      for (int e = 0; e < 8; e++) dst[e] = float4{x[4 * e], x[4 * e + 1], x[4 * e + 2], x[4 * e + 3]};
    }
    if (cmpl) {
      // F P from the rows of F still in registers (16 lanes per row)
      __syncthreads();  // P is complete
      for (int col = 0; col < p; col++) {
        float pv[8];
#pragma unroll
        for (int t = 0; t < 8; t++) pv[t] = Pg[(size_t)col * D + lane * 8 + t];
#pragma unroll
        for (int qq = 0; qq < NR; qq++) {
          float s = 0.f;
#pragma unroll
          for (int t = 0; t < 8; t++) s += f[qq][t] * pv[t];
          s = sum16(s);
          const int i = grp + NGR * qq;
          if (lane == 0 && i < b) YFP[i * D + k + col] = s;
        }
      }
    }
  }
  __syncthreads();

  // ---------------- phase B: R of Z, as R^T in the Jacobi layout -----------
  // Z = [diag(sigma) 0; FB FP]: its first k rows are already triangular, so
  // R comes from one structured QR step that folds the b block rows into
  // R_0 = [diag(sigma) 0; 0 0] (tsqr_core).
  float *J = smem;  // c columns (the rows of R), stride sj
  for (int idx = tid; idx < c * sj; idx += NTF) {
    const int col = idx / sj, row = idx - col * sj;
    J[idx] = (row == col && col < k) ? sig_old[col] : 0.f;
  }
  __syncthreads();
  tsqr_core<8 * NR>(J, sj, c, b, YFP, part, tau);

  // ---------------- phase C: one-sided Jacobi on the rows of R -------------
  double negl;
  {
    float fr = 0.f;
    for (int idx = tid; idx < c * sj; idx += NTF) fr += J[idx] * J[idx];
    fr = sum64(fr);
    if ((tid & 63) == 0) part[tid >> 6] = fr;
    __syncthreads();
    float fro2 = 0.f;
    for (int w = 0; w < NTF / 64; w++) fro2 += part[w];
    // Dot products in fp64: a pair is rotated while its cosine exceeds
    // 8 * 2^-24, just above what rotating fp32 columns can reach; columns
    // below c * 2^-24 * ||R|| are rounding noise and never rotated.
    const double tol = 8.0 * 5.9604644775390625e-8;
    const float ntol = (float)c * 5.9604645e-8f;
    negl = (double)(ntol * ntol * fro2);
    __syncthreads();  // part is reused below
    int sweep = 0;
    bool conv = (c < 2);
    switch (fold_nq(c)) {
      case 1: run_jacobi<1>(J, nrm, sj, c, tol, negl, sweep, conv); break;
      case 2: run_jacobi<2>(J, nrm, sj, c, tol, negl, sweep, conv); break;
      case 3: run_jacobi<3>(J, nrm, sj, c, tol, negl, sweep, conv); break;
      default: run_jacobi<4>(J, nrm, sj, c, tol, negl, sweep, conv); break;
    }
    if (tid == 0) {
      if (!conv) atomicOr(a.status, FLAG_SWEEP_CAP);
      X.sweeps[u] = sweep;
    }
  }

  // ---------------- phase D: sort, H, sign, B+, H_top, new rows -----------
  if (tid < k) tau[tid] = sig_old[tid];  // tau is dead after phase B; sigma is rewritten below
  {
    const int o = tid & 7, gid = tid >> 3;
    for (int col = gid; col < c; col += NTF / 8) {
      const float *zc = J + (size_t)col * sj + o * 4 * fold_nq(c);
      double s = 0.0;
      for (int e = 0; e < 4 * fold_nq(c); e++) s = fma((double)zc[e], (double)zc[e], s);
      s = octet_sum_d(s);
      if (o == 0) sv[col] = (float)sqrt(s);
    }
  }
  __syncthreads();
  // non-finite singular values are flagged and ranked last, so that perm
  // stays a permutation
  float me = 0.f;
  if (tid < c) {
    me = sv[tid];
    if (!(me <= 3.0e38f)) {
      atomicOr(a.status, FLAG_NONFINITE);
      me = -1.f;
    }
  }
  __syncthreads();
  if (tid < c) sv[tid] = me;
  __syncthreads();
  if (tid < c) {
    int rank = 0;
    for (int i = 0; i < c; i++) {
      const float o = sv[i];
      rank += (o > me || (o == me && i < tid)) ? 1 : 0;
    }
    perm[rank] = tid;
  }
  __syncthreads();
  if (tid == 0) {
    float dsum = 0.f;
    for (int qq = kplus; qq < c; qq++) dsum += sv[perm[qq]] * sv[perm[qq]];
    X.disc[u] = dsum;
  }
  // H = the converged columns over their norms (columns at the rounding level
  // are completed below)
  float *H = J;
  const float neglf = (float)negl;
  for (int idx = tid; idx < c * sj; idx += NTF) {
    const int col = idx / sj;
    const float s = sv[col];
    H[idx] = (s * s > neglf) ? H[idx] / s : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    // kept columns at the rounding level: the first unit vector e_t that keeps
    // a norm above 1/2 after two Gram-Schmidt passes against the other kept
    // columns (one wave, lanes hold rows ln and ln + 64)
    const int ln = tid;
    int t_next = 0;
    for (int jr = 0; jr < kplus; jr++) {
      const int cj = perm[jr];
      if (sv[cj] * sv[cj] > neglf) continue;
      for (; t_next < c; t_next++) {
        float w0 = (ln == t_next) ? 1.f : 0.f, w1 = (ln + 64 == t_next) ? 1.f : 0.f;
        for (int pass = 0; pass < 2; pass++) {
          for (int i = 0; i < kplus; i++) {
            if (i == jr) continue;
            const float *hc = H + (size_t)perm[i] * sj;
            const float b0 = (ln < c) ? hc[ln] : 0.f, b1 = (ln + 64 < c) ? hc[ln + 64] : 0.f;
            const float pr = sum64(w0 * b0 + w1 * b1);
            w0 -= pr * b0;
            w1 -= pr * b1;
          }
        }
        const float nn = sqrtf(sum64(w0 * w0 + w1 * w1));
        if (nn > 0.5f) {
          float *hc = H + (size_t)cj * sj;
          if (ln < c) hc[ln] = w0 / nn;
          if (ln + 64 < c) hc[ln + 64] = w1 / nn;
          t_next++;
          break;
        }
      }
    }
  }
  __syncthreads();

  // B+ = [B P] H_r into the second region (rows j' x D), 64 rows at a time
  float *Bp = smem + (size_t)c * sj;
  {
    const int cq = tid & 31;  // columns 4cq .. 4cq+3
    const int rg = tid >> 5;  // rows rg, rg+16, rg+32, rg+48 of each chunk
    for (int j0 = 0; j0 < kplus; j0 += 64) {
      float acc[4][4];
#pragma unroll
      for (int z = 0; z < 4; z++)
#pragma unroll
        for (int t = 0; t < 4; t++) acc[z][t] = 0.f;
      for (int i0 = 0; i0 < c; i0 += 8) {
        float4 bp[8];  // eight rows of [B; P] in flight at once
#pragma unroll
        for (int ii = 0; ii < 8; ii++) {
          const int i = i0 + ii;
          bp[ii] = float4{0.f, 0.f, 0.f, 0.f};
          if (i < c) {
            const float *src = (i < k) ? (Bt + (size_t)i * D) : (Pg + (size_t)(i - k) * D);
            bp[ii] = *reinterpret_cast<const float4 *>(src + 4 * cq);
          }
        }
#pragma unroll
        for (int ii = 0; ii < 8; ii++) {
          const int i = i0 + ii;
          if (i < c) {
#pragma unroll
            for (int z = 0; z < 4; z++) {
              const int jr = j0 + rg + 16 * z;
              if (jr < kplus) {
                const float hv = H[(size_t)perm[jr] * sj + i];
                acc[z][0] += hv * bp[ii].x;
                acc[z][1] += hv * bp[ii].y;
                acc[z][2] += hv * bp[ii].z;
                acc[z][3] += hv * bp[ii].w;
              }
            }
          }
        }
      }
#pragma unroll
      for (int z = 0; z < 4; z++) {
        const int jr = j0 + rg + 16 * z;
        if (jr < kplus)
          *reinterpret_cast<float4 *>(Bp + (size_t)jr * D + 4 * cq) = float4{acc[z][0], acc[z][1], acc[z][2], acc[z][3]};
      }
    }
  }
  __syncthreads();
  // sign rule: entry of largest magnitude (lowest index on ties) positive
  for (int jr = grp; jr < kplus; jr += NGR) {
    float best = -1.f;
    int bi = 0;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const float v = fabsf(Bp[(size_t)jr * D + lane * 8 + t]);
      if (v > best) {
        best = v;
        bi = lane * 8 + t;
      }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bi, off);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (lane == 0) sgn[jr] = (Bp[(size_t)jr * D + bi] < 0.f) ? -1.f : 1.f;
  }
  __syncthreads();
  // Re-orthonormalization (as in the fixed-coordinate core): with
  //   E = B+ B+^T - I and E_H = H_r^T H_r - I,
  // the basis becomes (I - E/2) B+ and the coordinates take G = I + E/2 - E_H
  // (a rotation error inflates C+ = Z H_r and B+ alike and is removed from
  // both; a basis error belongs to the coordinates), so C+ B+ is unchanged to
  // O(E^2) and sigma stays the column norms of the stored coordinates.
  for (int idx = tid; idx < kplus * D; idx += NTF) Bp[idx] *= sgn[idx / D];
  __syncthreads();
  float *Eg = Pg;                          // kplus x kplus: E
  float *Gg = Pg + (size_t)kplus * kplus;  // kplus x kplus: E/2 - E_H
  // both Gram matrices are symmetric (each entry's sums run in an order
  // symmetric in i and j), so one triangle is computed and mirrored
  for (int e = tid; e < kplus * (kplus + 1) / 2; e += NTF) {
    int i, j;
    tri_index(e, j, i);  // i <= j
    const float *bi = Bp + (size_t)i * D, *bj = Bp + (size_t)j * D;
    double acc = 0.0;
#pragma unroll 2
    for (int t = 0; t < D / 4; t++) {
      const int v = 4 * ((t + i + j) & (D / 4 - 1));  // rotate the start: fewer bank conflicts
      const float4 x = *reinterpret_cast<const float4 *>(bi + v);
      const float4 y = *reinterpret_cast<const float4 *>(bj + v);
      acc += (double)x.x * y.x + (double)x.y * y.y + (double)x.z * y.z + (double)x.w * y.w;
    }
    const float *hi = H + (size_t)perm[i] * sj, *hj = H + (size_t)perm[j] * sj;
    double ah = 0.0;
    for (int l = 0; l < c; l++) ah += (double)hi[l] * hj[l];
    ah *= (double)(sgn[i] * sgn[j]);
    const double dl = (i == j) ? 1.0 : 0.0;
    const float ev = (float)(acc - dl), gv = (float)(0.5 * (acc - dl) - (ah - dl));
    Eg[(size_t)i * kplus + j] = ev;
    Eg[(size_t)j * kplus + i] = ev;
    Gg[(size_t)i * kplus + j] = gv;
    Gg[(size_t)j * kplus + i] = gv;
  }
  __syncthreads();
  {
    // B = (I - E/2) B+ straight to the output basis; lanes own columns, so
    // every E entry a wave reads is uniform across it
    const int wv = tid >> 6, ln = tid & 63;
    constexpr int NW = NTF / 64;
    float *Btw = X.Bt + (size_t)u * r * D;
    for (int i0 = 4 * wv; i0 < kplus; i0 += 4 * NW) {
      float acc[4][2];
#pragma unroll
      for (int z = 0; z < 4; z++) acc[z][0] = acc[z][1] = 0.f;
      for (int l = 0; l < kplus; l++) {
        const float b0 = Bp[(size_t)l * D + ln], b1 = Bp[(size_t)l * D + ln + 64];
#pragma unroll
        for (int z = 0; z < 4; z++) {
          const float ev = (i0 + z < kplus) ? Eg[(size_t)(i0 + z) * kplus + l] : 0.f;
          acc[z][0] += ev * b0;
          acc[z][1] += ev * b1;
        }
      }
#pragma unroll
      for (int z = 0; z < 4; z++) {
        const int i = i0 + z;
        if (i < kplus) {
          Btw[(size_t)i * D + ln] = Bp[(size_t)i * D + ln] - 0.5f * acc[z][0];
          Btw[(size_t)i * D + ln + 64] = Bp[(size_t)i * D + ln + 64] - 0.5f * acc[z][1];
        }
      }
    }
    for (int idx = kplus * D + tid; idx < r * D; idx += NTF) Btw[idx] = 0.f;
  }
  __syncthreads();  // B+ in the second region is dead from here on
  // Hn = H_r G, signs and rank order applied, column-major (stride sj)
  float *Hn = Bp;
  {
    const int wv = tid >> 6, ln = tid & 63;
    constexpr int NW = NTF / 64;
    for (int j0 = 4 * wv; j0 < kplus; j0 += 4 * NW) {
      for (int i = ln; i < c; i += 64) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int l = 0; l < kplus; l++) {
          const float hv = sgn[l] * H[(size_t)perm[l] * sj + i];
#pragma unroll
          for (int z = 0; z < 4; z++)
            if (j0 + z < kplus) acc[z] += hv * Gg[(size_t)l * kplus + j0 + z];
        }
#pragma unroll
        for (int z = 0; z < 4; z++) {
          const int jr = j0 + z;
          if (jr < kplus) Hn[(size_t)jr * sj + i] = sgn[jr] * H[(size_t)perm[jr] * sj + i] + acc[z];
        }
      }
    }
  }
  __syncthreads();
  {
    float *Ht = X.Htop + (size_t)u * r * r;
    for (int idx = tid; idx < k * kplus; idx += NTF) {
      const int i = idx / kplus, jr = idx - i * kplus;
      Ht[(size_t)i * r + jr] = Hn[(size_t)jr * sj + i];
    }
  }
  // new rows C[n + i] = [F B | F P]_i Hn (b x k+), staged through the H region
  float *Ys = H;  // b x c, row stride c (b * c <= c * sj)
  for (int idx = tid; idx < b * c; idx += NTF) {
    const int i = idx / c, l = idx - i * c;
    Ys[idx] = YFP[(size_t)i * D + l];
  }
  __syncthreads();
  // Each thread owns one column and a strided set of rows, so the squared
  // column norms of the new rows reduce in a fixed order.
  const int ngrp = NTF / r;
  {
    TC *Cn = (TC *)X.C + (size_t)u * X.cstride + (size_t)a.n * r;
    if (tid < ngrp * r) {
      const int jr = tid % r, g0 = tid / r;
      float sq = 0.f;
      for (int i = g0; i < b; i += ngrp) {
        float s = 0.f;
        if (jr < kplus) {
          const float *hc = Hn + (size_t)jr * sj;
          const float *yr = Ys + (size_t)i * c;
          for (int l = 0; l < c; l++) s += yr[l] * hc[l];
        }
        stf<TC>(Cn, (size_t)i * r + jr, s);
        sq += s * s;
      }
      part[g0 * r + jr] = sq;
    }
  }
  __syncthreads();
  // sigma = column norms of the stored coordinates: rewritten old rows
  // (orthogonal columns of norms sigma_old, so sum_l sigma_l^2 Hn[l][j]^2)
  // plus the new rows. Computing it from what is stored keeps the next
  // fold's Z an exact description of the stored history.
  if (tid < r) {
    float s2 = 0.f;
    if (tid < kplus) {
      const float *hc = Hn + (size_t)tid * sj;
      for (int l = 0; l < k; l++) s2 += (tau[l] * hc[l]) * (tau[l] * hc[l]);
      for (int g = 0; g < ngrp; g++) s2 += part[g * r + tid];
    }
    X.sig[(size_t)u * r + tid] = sqrtf(s2);
  }
}

template <int NR, typename TK, typename TC>
__global__ void __launch_bounds__(NTF) __attribute__((amdgpu_waves_per_eu(2, 2))) k_fold(const FoldArgs a) {
  extern __shared__ float smem[];
  if (blockIdx.y == 0)
    fold_body<NR, TK, TC, 0>(a, smem);
  else
    fold_body<NR, TK, TC, 1>(a, smem);
}

template <int NR, typename TK, typename TC>
hipError_t launch_fold_t(const FoldArgs &a, int nunits, hipStream_t s) {
  size_t lds = fold_core_lds_bytes(a.k[0], a.b, a.r[0]);
  const size_t lv = fold_core_lds_bytes(a.k[1], a.b, a.r[1]);
  if (lv > lds) lds = lv;
  auto kern = k_fold<NR, TK, TC>;
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nunits, 2), dim3(NTF), lds, s, a);
  return hipGetLastError();
}

template <typename TK, typename TC>
hipError_t launch_fold_nr(const FoldArgs &a, int nunits, hipStream_t s) {
  const int nr = (a.b + NTF / 16 - 1) / (NTF / 16);
  if (nr <= 1) return launch_fold_t<1, TK, TC>(a, nunits, s);
  if (nr <= 2) return launch_fold_t<2, TK, TC>(a, nunits, s);
  return launch_fold_t<4, TK, TC>(a, nunits, s);
}

}  // namespace

size_t fold_core_lds_bytes(int k, int b, int r) { return sizeof(float) * (size_t)fold_lds(k, b, r).total; }

hipError_t launch_fold(const FoldArgs &a, int nunits, int kv_bf16, int coord_bf16, hipStream_t s) {
  if (kv_bf16 && coord_bf16) return launch_fold_nr<uint16_t, uint16_t>(a, nunits, s);
  if (kv_bf16 && !coord_bf16) return launch_fold_nr<uint16_t, float>(a, nunits, s);
  if (!kv_bf16 && coord_bf16) return launch_fold_nr<float, uint16_t>(a, nunits, s);
  return launch_fold_nr<float, float>(a, nunits, s);
}

}  // namespace iskv
