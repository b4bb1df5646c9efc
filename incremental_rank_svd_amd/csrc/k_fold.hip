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
#include <type_traits>

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
  // [B | E^T] as rows; when k + b >= d, B and then the projector I - B^T B
  // in rows 0 .. d-1 and F in rows d .. d+b-1
  const int a = (k + b >= D ? D + b : m) * LDA;
  const int h = c * sj;                    // R^T / H
  const int bp = kp * (LDA > sj ? LDA : sj);  // B+ staging (stride LDA), then H_r G (stride sj)
  int big = a;
  if (h + bp > big) big = h + bp;
  L.big = (big + 3) / 4 * 4;
  L.small = SMALL_FLOATS;
  L.total = L.big + L.small;
  return L;
}

template <int NQ>
__device__ __forceinline__ void run_jacobi(float *J, double *nrm, int sj, int c, double tol, double negl,
                                           int &sweep, bool &conv, uint32_t *flags, uint32_t *rmask, int *red) {
  jacobi_columns<NTF, LPJ, NQ>(J, nrm, sj, c, tol, negl, sweep, conv, flags, rmask, red);
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
  constexpr int NW = NTF / 64;  // wavefronts

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
  // When k + b >= d the residual basis has p = d - k columns: it is any
  // orthonormal basis of the complement of B (the residual rows lie in it),
  // so it comes from the QR of B alone and E is not needed.
  const bool cmpl = (k + b >= D);
  const int nref = cmpl ? k : c;  // reflectors that define P
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
  // F's rows in LDS rows d .. d+b-1 when k + b >= d (both of their products,
  // F B here and F P below, run on matrix cores)
  float *Fs = A + (size_t)D * LDA;
  if (cmpl) {
#pragma unroll
    for (int qq = 0; qq < NR; qq++) {
      const int i = grp + NGR * qq;
      if (i < b) {
#pragma unroll
        for (int t = 0; t < 8; t++) Fs[(size_t)i * LDA + lane * 8 + t] = f[qq][t];
      }
    }
  }
  __syncthreads();
  if (cmpl) {
    // Y = F B
    mfma_gemm_f32<NW>(
        b, k, D, [&](int i, int d) { return i < b ? Fs[(size_t)i * LDA + d] : 0.f; },
        [&](int d, int j) { return j < k ? A[(size_t)j * LDA + d] : 0.f; },
        [&](int i, int j, float v) {
          if (i < b && j < k) YFP[(size_t)i * D + j] = v;
        });
  } else {
    // Y = F B and E = F - Y B^T; then once more E <- E - (E B) B^T
    for (int pass = 0; pass < 2; pass++) {
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
#pragma unroll
          for (int t = 0; t < 8; t++) f[qq][t] -= s * bj[t];
          const int i = grp + NGR * qq;
          if (pass == 0 && lane == 0 && i < b) YFP[i * D + j] = s;
        }
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

  if (p > 0 && cmpl && p < k) {
    // P = an orthonormal basis of the complement of B (p = d - k < k): pivoted
    // Cholesky of the projector M = I - B^T B, p steps (fewer than the k
    // reflectors of a QR of B), M = G G^T. Since
    // G G^T = P^T P for any such basis, the columns of G are one: g_s is row
    // s of P. Step s pivots on the largest remaining diagonal (lowest index
    // on ties), which is at least 1/d in exact arithmetic.
    float *M = A;  // d rows, stride LDA (B's rows are dead: Y = F B is done)
    {
      // M in fp64 on matrix cores (B from memory, a tile's operands loaded
      // before its products; one triangle of tiles, mirrored), rounded to fp32
      const int wv = tid >> 6, ln = tid & 63, l16 = ln & 15, lk = ln >> 4;
      constexpr int TD = D / 16;
      for (int t = wv; t < TD * (TD + 1) / 2; t += NW) {
        int tj, ti;
        tri_index(t, tj, ti);  // ti <= tj
        const int ia = 16 * ti + l16, jb = 16 * tj + l16;
        float x[D / 4], y[D / 4];
#pragma unroll
        for (int z = 0; z < D / 4; z++) {
          const int l = 4 * z + lk;
          x[z] = l < k ? Bt[(size_t)l * D + ia] : 0.f;
          y[z] = l < k ? Bt[(size_t)l * D + jb] : 0.f;
        }
        mf64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int z = 0; z < D / 4; z++)
          if (4 * z < k) acc = mfma4_f64((double)x[z], (double)y[z], acc);
#pragma unroll
        for (int v = 0; v < 4; v++) {
          const int i = 16 * ti + lk + 4 * v, j = jb;  // fp64 accumulator layout
          if (i <= j) {
            const float mv = (float)((i == j ? 1.0 : 0.0) - acc[v]);
            M[(size_t)i * LDA + j] = mv;
            M[(size_t)j * LDA + i] = mv;
          }
        }
      }
    }
    // indices not yet pivots: a 128-bit mask, the same in every thread
    uint32_t am[4] = {~0u, ~0u, ~0u, ~0u};
    auto active = [&](int i) -> bool {
      const uint32_t w = i < 64 ? (i < 32 ? am[0] : am[1]) : (i < 96 ? am[2] : am[3]);
      return (w >> (i & 31)) & 1u;
    };
    float *g = sv;
    __syncthreads();
    for (int st = 0; st < p; st++) {
      if (tid < 64) {
        float bv = -1.f;
        int bi = 0;
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int i = tid + 64 * h;
          const float dv = active(i) ? M[(size_t)i * LDA + i] : -1.f;
          if (dv > bv) {
            bv = dv;
            bi = i;
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oi = __shfl_xor(bi, off);
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (tid == 0) {
          ((int *)part)[0] = bi;
          part[1] = bv;
        }
      }
      __syncthreads();
      const int piv = ((const int *)part)[0];
      if (tid < D) {
        const float rs = 1.f / sqrtf(fmaxf(part[1], 1e-30f));
        const float gv = active(tid) ? M[(size_t)tid * LDA + piv] * rs : 0.f;
        g[tid] = gv;
        Pg[(size_t)st * D + tid] = gv;
      }
      am[piv >> 5] &= ~(1u << (piv & 31));
      __syncthreads();
      // M <- M - g g^T on the columns that are not pivots yet (rows that are
      // pivots have g = 0, except this step's, which is never read again)
      {
        const int j = tid & (D - 1), i0 = tid >> 7;
        if (active(j)) {
          const float gj = g[j];
#pragma unroll 8
          for (int q = 0; q < D / (NTF / D); q++) {
            const int i = i0 + (NTF / D) * q;
            M[(size_t)i * LDA + j] -= g[i] * gj;
          }
        }
      }
      __syncthreads();
    }
    // F P, F from LDS rows d .. d+b-1
    mfma_gemm_f32<NW>(
        b, p, D, [&](int i, int d) { return i < b ? Fs[(size_t)i * LDA + d] : 0.f; },
        [&](int d, int col) { return col < p ? Pg[(size_t)col * D + d] : 0.f; },
        [&](int i, int col, float v) {
          if (i < b && col < p) YFP[(size_t)i * D + k + col] = v;
        });
  } else if (p > 0) {
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
      // F P, F from LDS rows d .. d+b-1
      __syncthreads();  // P is complete
      mfma_gemm_f32<NW>(
          b, p, D, [&](int i, int d) { return i < b ? Fs[(size_t)i * LDA + d] : 0.f; },
          [&](int d, int col) { return col < p ? Pg[(size_t)col * D + d] : 0.f; },
          [&](int i, int col, float v) {
            if (i < b && col < p) YFP[(size_t)i * D + k + col] = v;
          });
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
    // Jacobi scratch: the pair flags in tau .. perm (dead until phase D, 4 D
    // words >= c ceil(c/32)), the round mask and a counter in part
    uint32_t *flags = (uint32_t *)tau;
    uint32_t *rmask = (uint32_t *)part;
    int *red = (int *)(part + 4);
    switch (fold_nq(c)) {
      case 1: run_jacobi<1>(J, nrm, sj, c, tol, negl, sweep, conv, flags, rmask, red); break;
      case 2: run_jacobi<2>(J, nrm, sj, c, tol, negl, sweep, conv, flags, rmask, red); break;
      case 3: run_jacobi<3>(J, nrm, sj, c, tol, negl, sweep, conv, flags, rmask, red); break;
      default: run_jacobi<4>(J, nrm, sj, c, tol, negl, sweep, conv, flags, rmask, red); break;
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

  // The products below run on matrix cores (fp32, the Gram matrices fp64).
  // B+ = [B P] H_r into the second region (rows j' x D, stride LDA)
  float *Bp = smem + (size_t)c * sj;
  mfma_gemm_f32<NW>(
      kplus, D, c,
      [&](int jr, int i) { return (jr < kplus && i < c) ? H[(size_t)perm[jr] * sj + i] : 0.f; },
      [&](int i, int d) {
        return i < c ? ((i < k) ? Bt[(size_t)i * D + d] : Pg[(size_t)(i - k) * D + d]) : 0.f;
      },
      [&](int jr, int d, float v) {
        if (jr < kplus) Bp[(size_t)jr * LDA + d] = v;
      });
  __syncthreads();
  // sign rule: entry of largest magnitude (lowest index on ties) positive
  for (int jr = grp; jr < kplus; jr += NGR) {
    float best = -1.f;
    int bi = 0;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const float v = fabsf(Bp[(size_t)jr * LDA + lane * 8 + t]);
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
    if (lane == 0) sgn[jr] = (Bp[(size_t)jr * LDA + bi] < 0.f) ? -1.f : 1.f;
  }
  __syncthreads();
  // Re-orthonormalization (as in the fixed-coordinate core): with
  //   E = B+ B+^T - I and E_H = H_r^T H_r - I,
  // the basis becomes (I - E/2) B+ and the coordinates take G = I + E/2 - E_H
  // (a rotation error inflates C+ = Z H_r and B+ alike and is removed from
  // both; a basis error belongs to the coordinates), so C+ B+ is unchanged to
  // O(E^2) and sigma stays the column norms of the stored coordinates.
  for (int idx = tid; idx < kplus * D; idx += NTF) Bp[(size_t)(idx / D) * LDA + idx % D] *= sgn[idx / D];
  __syncthreads();
  float *Eg = Pg;                          // kplus x kplus: E
  float *Gg = Pg + (size_t)kplus * kplus;  // kplus x kplus: E/2 - E_H
  {
    // both Gram matrices in fp64 on matrix cores, the tiles of one triangle
    // only: each entry is computed once and mirrored, so both are exactly
    // symmetric
    const int wv = tid >> 6, ln = tid & 63, l16 = ln & 15, lk = ln >> 4;
    const int tk = (kplus + 15) >> 4;
    for (int t = wv; t < tk * (tk + 1) / 2; t += NW) {
      int tj, ti;
      tri_index(t, tj, ti);  // ti <= tj
      const int ia = 16 * ti + l16, jb = 16 * tj + l16;
      const bool va = ia < kplus, vb = jb < kplus;
      const float *ra = Bp + (size_t)(va ? ia : 0) * LDA, *rb = Bp + (size_t)(vb ? jb : 0) * LDA;
      mf64x4 e = {0.0, 0.0, 0.0, 0.0}, h = {0.0, 0.0, 0.0, 0.0};
      for (int d0 = 0; d0 < D; d0 += 16) {
        double x[4], y[4];
#pragma unroll
        for (int z = 0; z < 4; z++) {
          x[z] = va ? (double)ra[d0 + 4 * z + lk] : 0.0;
          y[z] = vb ? (double)rb[d0 + 4 * z + lk] : 0.0;
        }
#pragma unroll
        for (int z = 0; z < 4; z++) e = mfma4_f64(x[z], y[z], e);
      }
      const float *ha = H + (size_t)perm[va ? ia : 0] * sj, *hb = H + (size_t)perm[vb ? jb : 0] * sj;
      for (int l0 = 0; l0 < c; l0 += 16) {
        double x[4], y[4];
#pragma unroll
        for (int z = 0; z < 4; z++) {
          const int l = l0 + 4 * z + lk;
          x[z] = (va && l < c) ? (double)ha[l] : 0.0;
          y[z] = (vb && l < c) ? (double)hb[l] : 0.0;
        }
#pragma unroll
        for (int z = 0; z < 4; z++) h = mfma4_f64(x[z], y[z], h);
      }
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int i = 16 * ti + lk + 4 * v, j = jb;  // fp64 accumulator layout
        if (i < kplus && j < kplus && i <= j) {
          const double dl = (i == j) ? 1.0 : 0.0;
          const double ah = h[v] * (double)(sgn[i] * sgn[j]);
          const float ev = (float)(e[v] - dl), gv = (float)(0.5 * (e[v] - dl) - (ah - dl));
          Eg[(size_t)i * kplus + j] = ev;
          Eg[(size_t)j * kplus + i] = ev;
          Gg[(size_t)i * kplus + j] = gv;
          Gg[(size_t)j * kplus + i] = gv;
        }
      }
    }
  }
  __syncthreads();
  // B = (I - E/2) B+ straight to the output basis
  {
    float *Btw = X.Bt + (size_t)u * r * D;
    mfma_gemm_f32<NW>(
        kplus, D, kplus,
        [&](int i, int l) { return (i < kplus && l < kplus) ? Eg[(size_t)i * kplus + l] : 0.f; },
        [&](int l, int d) { return l < kplus ? Bp[(size_t)l * LDA + d] : 0.f; },
        [&](int i, int d, float v) {
          if (i < kplus) Btw[(size_t)i * D + d] = Bp[(size_t)i * LDA + d] - 0.5f * v;
        });
    for (int idx = kplus * D + tid; idx < r * D; idx += NTF) Btw[idx] = 0.f;
  }
  __syncthreads();  // B+ in the second region is dead from here on
  // Hn = H_r G, signs and rank order applied, column-major (stride sj)
  float *Hn = Bp;
  mfma_gemm_f32<NW>(
      c, kplus, kplus,
      [&](int i, int l) { return (i < c && l < kplus) ? sgn[l] * H[(size_t)perm[l] * sj + i] : 0.f; },
      [&](int l, int jr) { return (l < kplus && jr < kplus) ? Gg[(size_t)l * kplus + jr] : 0.f; },
      [&](int i, int jr, float v) {
        if (i < c && jr < kplus) Hn[(size_t)jr * sj + i] = sgn[jr] * H[(size_t)perm[jr] * sj + i] + v;
      });
  __syncthreads();
  constexpr bool I8 = std::is_same<TC, int8_t>::value;
  if constexpr (!I8) {
    float *Ht = X.Htop + (size_t)u * r * r;
    for (int idx = tid; idx < k * kplus; idx += NTF) {
      const int i = idx / kplus, jr = idx - i * kplus;
      Ht[(size_t)i * r + jr] = Hn[(size_t)jr * sj + i];
    }
  }
  // new rows C[n + i] = [F B | F P]_i Hn (b x r, columns k+ .. r-1 zero). The
  // squared column norms of each 16-row tile go to sqp (the small arrays from
  // sv on, dead by now: ceil(b/16) r <= 1024 floats) and are summed in a
  // fixed order below.
  float *sqp = sv;
  {
    TC *Cn = (TC *)X.C + (size_t)u * X.cstride + (size_t)a.n * r;
    const int ln = tid & 63, l16 = ln & 15, lk = ln >> 4;
    mfma_gemm_tiles_f32<NW>(
        b, r, c,
        [&](int i, int l) { return (i < b && l < c) ? YFP[(size_t)i * D + l] : 0.f; },
        [&](int l, int jr) { return (l < c && jr < kplus) ? Hn[(size_t)jr * sj + l] : 0.f; },
        [&](int i0, int j0, mf32x4 acc) {
          const int jr = j0 + l16;
          float sq = 0.f;
#pragma unroll
          for (int v = 0; v < 4; v++) {
            const int i = i0 + 4 * lk + v;
            if constexpr (I8) {
              // int8 storage needs the new sigma first: the rows wait in the
              // fold scratch (free since H_r G)
              if (i < b && jr < r) Pg[(size_t)i * r + jr] = acc[v];
            } else {
              if (i < b && jr < r) stf<TC>(Cn, (size_t)i * r + jr, acc[v]);
            }
            sq += acc[v] * acc[v];  // zero for rows past b
          }
          sq += __shfl_xor(sq, 16);
          sq += __shfl_xor(sq, 32);
          if (lk == 0 && jr < r) sqp[(i0 >> 4) * r + jr] = sq;
        });
  }
  __syncthreads();
  // sigma = column norms of the stored coordinates: rewritten old rows
  // (orthogonal columns of norms sigma_old, so sum_l sigma_l^2 Hn[l][j]^2)
  // plus the new rows. Computing it from what is stored keeps the next
  // fold's Z an exact description of the stored history.
  float *sgnew = smem;  // H's region, dead since H_r G: the new sigma for int8 storage
  if (tid < r) {
    float s2 = 0.f;
    if (tid < kplus) {
      const float *hc = Hn + (size_t)tid * sj;
      for (int l = 0; l < k; l++) s2 += (tau[l] * hc[l]) * (tau[l] * hc[l]);
      for (int mt = 0; mt < (b + 15) / 16; mt++) s2 += sqp[mt * r + tid];
    }
    X.sig[(size_t)u * r + tid] = sqrtf(s2);
    if constexpr (I8) {
      if (tid < kplus) sgnew[tid] = sqrtf(s2);  // kplus <= c floats, below H_r G at c * sj
    }
  }
  if constexpr (I8) {
    // int8 storage keeps U = C Sigma^-1. The stored rows of U rotate by
    // M = Sigma_old H_top Sigma_new^-1 (C_old H_top = U_old M Sigma_new); the
    // new rows of U are the new rows of C over the new sigma, each stored as
    // int8 codes with its own scale (max|u| / 127). A column with sigma 0 is
    // zero in C, so its U column is written as zero.
    __syncthreads();
    float *Ht = X.Htop + (size_t)u * r * r;
    for (int idx = tid; idx < k * kplus; idx += NTF) {
      const int i = idx / kplus, jr = idx - i * kplus;
      const float sn = sgnew[jr];
      Ht[(size_t)i * r + jr] = sn > 0.f ? tau[i] * Hn[(size_t)jr * sj + i] / sn : 0.f;
    }
    int8_t *Cn = (int8_t *)X.C + (size_t)u * X.cstride + (size_t)a.n * r;
    float *cs = X.cs + (size_t)u * cs_stride(a.ncap) + a.n;
    const int wv = tid >> 6, ln = tid & 63;
    for (int i = wv; i < b; i += NW) {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int j = ln + 64 * h;
        const float sn = j < kplus ? sgnew[j] : 0.f;
        v[h] = sn > 0.f ? Pg[(size_t)i * r + j] / sn : 0.f;
      }
      const float m = max64(fmaxf(fabsf(v[0]), fabsf(v[1])));
      const float inv = i8_inv_step(m);
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int j = ln + 64 * h;
        if (j < r) Cn[(size_t)i * r + j] = (int8_t)i8_code(v[h], inv);
      }
      if (ln == 0) cs[i] = m / 127.f;
    }
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
  if (a.X[0].cs) return launch_fold_nr<uint16_t, int8_t>(a, nunits, s);  // int8 storage of U (bf16 rows)
  if (kv_bf16 && coord_bf16) return launch_fold_nr<uint16_t, uint16_t>(a, nunits, s);
  if (kv_bf16 && !coord_bf16) return launch_fold_nr<uint16_t, float>(a, nunits, s);
  if (!kv_bf16 && coord_bf16) return launch_fold_nr<float, uint16_t>(a, nunits, s);
  return launch_fold_nr<float, float>(a, nunits, s);
}

}  // namespace iskv
