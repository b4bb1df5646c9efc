// Fold core: one workgroup per unit, everything resident in LDS.
//
// Page "iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental
// SVD", section "Block-Incremental Decoding Updates":
//   1. residual E = F - (F B) B^T (orthogonalized twice against B) and a
//      residual basis P: here the Householder QR of the d x (k+b) matrix
//      [B | E^T]; P = Q[:, k:k+p], p = min(b, d-k), and F P is read off the
//      triangular factor (F P = R[k:k+p, k:k+b]^T).
//   2. core Z = [Sigma 0; FB FP], (k+b) x (k+p).
//   3. (G, Sigma+, H) = SVD_r(Z) by one-sided Jacobi with round-robin
//      parallel ordering (a QR of Z first when it has more rows than
//      columns), then B+ = [B P] H_r.
// The coordinate rewrite C+ = [C 0; FB FP] H_r (U+ Sigma+ without a division
// by sigma, since Z H = G Sigma) is split: this kernel writes the b new rows
// and H_top = H[0:k, 0:k+]; k_rewrite.hip streams the n old rows.
//
// Work mapping: quads (4 consecutive lanes) own one Jacobi pair, one
// Householder column or one column of P; their sums use two DPP quad
// permutations. Columns in LDS have a stride of 4 (mod 16) floats so that
// different columns start in different banks.
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int LDA = D + 4;  // LDS stride of the [B | E^T] columns (4 mod 32)
__host__ __device__ inline int ldz(int m) { return ((m + 31) / 32) * 32 + 4; }

// rows per quad lane of a Jacobi column (a multiple of 4) and column stride
__host__ __device__ inline int jac_rl(int c) { return 4 * ((c + 15) / 16); }
__host__ __device__ inline int jac_stride(int c) { return 4 * jac_rl(c) + 4; }

struct CoreLds {
  int a, z, j, h, total;  // floats: phase A, Z before its QR, J region, H region, max
};

__host__ __device__ inline CoreLds core_lds(int k, int b, int r) {
  CoreLds L;
  const int p = (b < D - k) ? b : D - k;
  const int m = k + b, c = k + p;
  const int kp = (r < c) ? r : c;
  const int sj = jac_stride(c);
  L.a = (k + b) * LDA;
  L.z = (m > c) ? ldz(m) * c : 0;
  int jr = c * sj;
  if (kp * D > jr) jr = kp * D;  // B+ staging
  if (b * c > jr) jr = b * c;    // [FB FP] staging
  L.j = (jr + 3) / 4 * 4;  // H (float4 accesses) starts 16-byte aligned
  L.h = c * sj;
  int mx = L.a > L.z ? L.a : L.z;
  L.total = mx > L.j + L.h ? mx : L.j + L.h;
  return L;
}

// (column, row) of entry e of a column-major packed upper triangle
__device__ __forceinline__ void tri_index(int e, int &col, int &row) {
  int cc = (int)((sqrtf(8.f * (float)e + 1.f) - 1.f) * 0.5f);
  while (cc > 0 && cc * (cc + 1) / 2 > e) cc--;
  while ((cc + 1) * (cc + 2) / 2 <= e) cc++;
  col = cc;
  row = e - cc * (cc + 1) / 2;
}

// pair (i < j) of round `rnd` in a round-robin over c2 players (c2 even)
__device__ __forceinline__ void rr_pair(int rnd, int pr, int c2, int &i, int &j) {
  int a, b;
  if (pr == 0) {
    a = rnd;
    b = c2 - 1;
  } else {
    const int mdl = c2 - 1;
    a = (rnd + pr) % mdl;
    b = (rnd - pr + mdl) % mdl;
  }
  i = a < b ? a : b;
  j = a < b ? b : a;
}

// double-precision quad sum (two 32-bit DPP moves per step)
__device__ __forceinline__ double dpp_d(double v, int ctrl_xor1) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const int lo = (int)(u & 0xffffffffull), hi = (int)(u >> 32);
  int lo2, hi2;
  if (ctrl_xor1) {
    lo2 = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
    hi2 = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false);
  } else {
    lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
    hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false);
  }
  return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi2 << 32) | (unsigned)lo2);
}
__device__ __forceinline__ double quad_sum_d(double v) {
  v += dpp_d(v, 1);
  v += dpp_d(v, 0);
  return v;
}

// sum over the 4 lanes of a quad (DPP quad permutations, no LDS traffic)
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  return v;
}

// Householder QR (LAPACK dlarfg convention: H = I - tau v v^T, v[0] = 1,
// H x = beta e_0) of an nrows x ncols matrix stored column-major in LDS with
// column stride ld; nref reflectors. On return the upper triangle holds R,
// the part below the diagonal v (without its unit head) and tau[j] the
// scalars. Quad qid owns the columns qid, qid + 64, ...; lane q of a quad
// holds rows q, q+4, q+8, ... (consecutive lanes, consecutive words). The
// owner of column j+1 builds reflector j+1 as soon as it has applied
// reflector j (one barrier per reflector). ld should be 4 mod 32 so that the
// columns of different quads start in different banks.
template <int RQ, bool FULL>
__device__ __forceinline__ void house_qr(float *A, int ld, int nrows, int ncols, int nref, float *tau) {
  // FULL: nrows == 4 RQ, so every row q + 4e exists. Then every load and
  // store is unconditional (masking is arithmetic: v is zero above the
  // diagonal, rows above it are written back unchanged), which lets a lane
  // issue all RQ loads of a column back to back instead of one per branch.
  const int tid = threadIdx.x, q = tid & 3, qid = tid >> 2;
  auto inrange = [&](int row) { return FULL || row < nrows; };
  auto reflector = [&](int j) {
    float *cj = A + (size_t)j * ld;
    float s = 0.f;
    float x[RQ];
#pragma unroll
    for (int e = 0; e < RQ; e++) {
      const int row = q + 4 * e;
      x[e] = 0.f;
      if (FULL) {
        x[e] = cj[row];
      } else if (row < nrows) {
        x[e] = cj[row];
      }
      const float t = (row > j && inrange(row)) ? x[e] : 0.f;
      s += t * t;
    }
    s = quad_sum(s);
    const float x0 = cj[j];
    float tj = 0.f, beta = x0, scal = 0.f;
    if (s > 0.f) {
      beta = -copysignf(sqrtf(x0 * x0 + s), x0);
      tj = (beta - x0) / beta;
      scal = 1.f / (x0 - beta);
    }
#pragma unroll
    for (int e = 0; e < RQ; e++) {
      const int row = q + 4 * e;
      if (FULL) {
        cj[row] = (row > j) ? x[e] * scal : ((row == j) ? beta : x[e]);
      } else {
        if (row > j && row < nrows) cj[row] = x[e] * scal;
        if (row == j) cj[j] = beta;
      }
    }
    if (q == 0) tau[j] = tj;
  };
  if (nref > 0 && qid == 0) reflector(0);
  __syncthreads();
  for (int j = 0; j < nref; j++) {
    const float tj = tau[j];
    if (tj != 0.f) {
      const float *cj = A + (size_t)j * ld;
      float v[RQ];
#pragma unroll
      for (int e = 0; e < RQ; e++) {
        const int row = q + 4 * e;
        if (FULL) {
          const float cv = cj[row];
          v[e] = (row > j) ? cv : ((row == j) ? 1.f : 0.f);
        } else {
          v[e] = (row < nrows && row >= j) ? ((row == j) ? 1.f : cj[row]) : 0.f;
        }
      }
      int col = qid;
      while (col <= j) col += NT / 4;
      for (; col < ncols; col += NT / 4) {
        float *cc = A + (size_t)col * ld;
        if (FULL) {
          // column in registers: one pass of loads, one of stores
          float x[RQ];
          float w = 0.f;
#pragma unroll
          for (int e = 0; e < RQ; e++) {
            x[e] = cc[q + 4 * e];
            w += v[e] * x[e];
          }
          w = tj * quad_sum(w);
#pragma unroll
          for (int e = 0; e < RQ; e++) cc[q + 4 * e] = x[e] - w * v[e];
        } else {
          // two passes over the column (dot, then update): only v stays in registers
          float w = 0.f;
#pragma unroll
          for (int e = 0; e < RQ; e++) {
            const int row = q + 4 * e;
            if (row < nrows && row >= j) w += v[e] * cc[row];
          }
          w = tj * quad_sum(w);
#pragma unroll
          for (int e = 0; e < RQ; e++) {
            const int row = q + 4 * e;
            if (row < nrows && row >= j) cc[row] -= w * v[e];
          }
        }
      }
    }
    if (j + 1 < nref && qid == ((j + 1) & (NT / 4 - 1))) reflector(j + 1);
    __syncthreads();
  }
}

// Cyclic sweeps of one-sided Jacobi over the columns of J (c columns, column
// stride sj, rows split over the 4 lanes of a quad, NQ float4 chunks per
// lane), accumulating the same rotations in H. A quad owns one pair of the
// parallel round-robin order per round; cosines are measured from fp64 dot
// products. The squared column norms are kept in nrm (fp64): measured at the
// start of every sweep and carried through each rotation by its exact effect
// on the two norms, so a pair costs one dot product instead of three. Stops
// after a sweep without rotation or at SWEEP_CAP.
template <int NQ>
__device__ __forceinline__ void jacobi_sweeps(float *J, float *H, double *nrm, int sj, int rl, int c, int c2,
                                              double tol, double negl, int &sweep, bool &conv) {
  const int tid = threadIdx.x, q = tid & 3, qid = tid >> 2;
  while (!conv && sweep < SWEEP_CAP) {
    sweep++;
    int rot = 0;
    for (int col = qid; col < c; col += NT / 4) {
      const float4 *zc = (const float4 *)(J + (size_t)col * sj + q * rl);
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int e = 0; e < NQ; e++) {
        const float4 x = zc[e];
        s0 = fma((double)x.x, (double)x.x, s0);
        s1 = fma((double)x.y, (double)x.y, s1);
        s0 = fma((double)x.z, (double)x.z, s0);
        s1 = fma((double)x.w, (double)x.w, s1);
      }
      const double sn2 = quad_sum_d(s0 + s1);
      if (q == 0) nrm[col] = sn2;
    }
    __syncthreads();
    for (int rnd = 0; rnd < c2 - 1; rnd++) {
      if (qid < c2 / 2) {
        int ci, cj;
        rr_pair(rnd, qid, c2, ci, cj);
        if (cj < c) {
          float4 *zi = (float4 *)(J + (size_t)ci * sj + q * rl);
          float4 *zj = (float4 *)(J + (size_t)cj * sj + q * rl);
          float4 xi[NQ], xj[NQ];
          const double al = nrm[ci], be = nrm[cj];
          double ga = 0.0, ga2 = 0.0;
#pragma unroll
          for (int e = 0; e < NQ; e++) {
            xi[e] = zi[e];
            xj[e] = zj[e];
          }
#pragma unroll
          for (int e = 0; e < NQ; e++) {
            // fma chains (one fp64 op per product), two for latency
            ga = fma((double)xi[e].x, (double)xj[e].x, ga);
            ga2 = fma((double)xi[e].y, (double)xj[e].y, ga2);
            ga = fma((double)xi[e].z, (double)xj[e].z, ga);
            ga2 = fma((double)xi[e].w, (double)xj[e].w, ga2);
          }
          ga = quad_sum_d(ga + ga2);
          if (al > negl && be > negl && ga * ga > tol * tol * (al * be)) {
            // The sums are fp64; the angle itself only needs fp32 (it is applied
            // to fp32 columns, and cs, sn are rounded to fp32 anyway).
            const float zeta = (float)(be - al) / (float)(2.0 * ga);
            const float az = fabsf(zeta);
            float t = (az > 1e18f) ? 0.5f / az : 1.f / (az + sqrtf(1.f + az * az));
            t = copysignf(t, zeta);
            const float cs = 1.f / sqrtf(1.f + t * t);
            const float sn = cs * t;
            float4 *hi = (float4 *)(H + (size_t)ci * sj + q * rl);
            float4 *hj = (float4 *)(H + (size_t)cj * sj + q * rl);
            float4 yi[NQ], yj[NQ];
#pragma unroll
            for (int e = 0; e < NQ; e++) {
              yi[e] = hi[e];
              yj[e] = hj[e];
            }
#pragma unroll
            for (int e = 0; e < NQ; e++) {
              const float4 u0 = xi[e], u1 = xj[e];
              zi[e] = float4{cs * u0.x - sn * u1.x, cs * u0.y - sn * u1.y, cs * u0.z - sn * u1.z,
                             cs * u0.w - sn * u1.w};
              zj[e] = float4{sn * u0.x + cs * u1.x, sn * u0.y + cs * u1.y, sn * u0.z + cs * u1.z,
                             sn * u0.w + cs * u1.w};
            }
#pragma unroll
            for (int e = 0; e < NQ; e++) {
              const float4 u0 = yi[e], u1 = yj[e];
              hi[e] = float4{cs * u0.x - sn * u1.x, cs * u0.y - sn * u1.y, cs * u0.z - sn * u1.z,
                             cs * u0.w - sn * u1.w};
              hj[e] = float4{sn * u0.x + cs * u1.x, sn * u0.y + cs * u1.y, sn * u0.z + cs * u1.z,
                             sn * u0.w + cs * u1.w};
            }
            if (q == 0) {
              // norms of the rotated pair, from the rotation actually applied
              const double c_ = cs, s_ = sn, cg = 2.0 * c_ * s_ * ga;
              nrm[ci] = fmax(c_ * c_ * al - cg + s_ * s_ * be, 0.0);
              nrm[cj] = fmax(s_ * s_ * al + cg + c_ * c_ * be, 0.0);
            }
            rot = 1;
          }
        }
      }
      __syncthreads();
    }
    conv = !__syncthreads_or(rot);
  }
}

// XK (0 keys, 1 values) is a template constant so that every access to the
// kernel arguments has a constant offset (a dynamic index would copy them to
// scratch memory).
template <int NR, typename TK, typename TC, int XK>
__device__ __forceinline__ void core_body(const FoldArgs &a, float *smem) {
  const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4;
  const int q = tid & 3, qid = tid >> 2;
  const int u = a.u0 + blockIdx.x;
  const Stream &X = a.X[XK];
  const int b = a.b, k = a.k[XK], r = a.r[XK];
  const int p = (b < D - k) ? b : D - k;
  const int m = k + b, c = k + p;
  const int kplus = (r < c) ? r : c;
  const int rl = jac_rl(c);      // J/H rows per quad lane
  const int sj = jac_stride(c);  // column stride of J and H
  const CoreLds lay = core_lds(k, b, r);

  float *tau = smem + a.lds_small[XK];
  float *sv = tau + D;
  float *sgn = sv + D;
  int *perm = (int *)(sgn + D);

  const float *Bt = X.Bt + (size_t)u * r * D;
  float *Pg = X.P + (size_t)u * a.pmax * D;
  float *YFP = X.YFP + (size_t)u * a.bmax * D;
  const TK *ring = (const TK *)X.ring + (size_t)u * a.rcap * D;

  // ---------------- phase A: projection, residual, residual basis ---------
  float *A = smem;  // rows 0..k-1 = basis vectors, rows k..k+b-1 = residual rows (stride LDA)
  // B into LDS, four float4 loads in flight per thread at a time
  for (int i0 = tid; i0 < k * (D / 4); i0 += 4 * NT) {
    float4 bq[4];
#pragma unroll
    for (int z = 0; z < 4; z++) {
      const int idx = i0 + NT * z;
      if (idx < k * (D / 4)) bq[z] = reinterpret_cast<const float4 *>(Bt)[idx];
    }
#pragma unroll
    for (int z = 0; z < 4; z++) {
      const int idx = i0 + NT * z;
      if (idx < k * (D / 4)) {
        const int row = idx / (D / 4), c4 = idx - row * (D / 4);
        *reinterpret_cast<float4 *>(A + (size_t)row * LDA + 4 * c4) = bq[z];
      }
    }
  }
  float f[NR][8];
#pragma unroll
  for (int qq = 0; qq < NR; qq++) {
    const int i = grp + 16 * qq;
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
        const int i = grp + 16 * qq;
        if (pass == 0 && lane == 0 && i < b) YFP[i * D + j] = s;
      }
    }
  }
#pragma unroll
  for (int qq = 0; qq < NR; qq++) {
    const int i = grp + 16 * qq;
    if (i < b) {
#pragma unroll
      for (int t = 0; t < 8; t++) A[(k + i) * LDA + lane * 8 + t] = f[qq][t];
    }
  }
  __syncthreads();

  if (p > 0) {
    // Householder QR of [B | E^T] (column j = LDS row j), c reflectors.
    house_qr<D / 4, true>(A, LDA, D, k + b, c, tau);
    // P = Q[:, k:k+p] = H_0 ... H_{c-1} [e_k .. e_{k+p-1}], accumulated backwards
    // in the registers of one quad per column (lane q: rows q, q+4, ...);
    // reflectors j > k+col leave e_{k+col} unchanged and are skipped.
    for (int col = qid; col < p; col += NT / 4) {
      float x[D / 4];
#pragma unroll
      for (int e = 0; e < D / 4; e++) x[e] = (q + 4 * e == k + col) ? 1.f : 0.f;
      for (int j = k + col; j >= 0; j--) {
        const float tj = tau[j];
        if (tj == 0.f) continue;
        const float *cj = A + (size_t)j * LDA;
        // reflector j as coefficients (v = 1 at row j, stored below it); all
        // D rows are loaded unconditionally and masked arithmetically
        float vj[D / 4];
        float w = 0.f;
#pragma unroll
        for (int e = 0; e < D / 4; e++) {
          const int row = q + 4 * e;
          const float cv = cj[row];
          vj[e] = (row > j) ? cv : ((row == j) ? 1.f : 0.f);
          w += vj[e] * x[e];
        }
        w = tj * quad_sum(w);
#pragma unroll
        for (int e = 0; e < D / 4; e++) x[e] -= w * vj[e];
      }
#pragma unroll
      for (int e = 0; e < D / 4; e++) Pg[(size_t)col * D + q + 4 * e] = x[e];
    }
    // F P = R[k:k+p, k:k+b]^T (lower trapezoidal)
    for (int idx = tid; idx < b * p; idx += NT) {
      const int i = idx / p, qq = idx - i * p;
      YFP[i * D + k + qq] = (qq <= i) ? A[(size_t)(k + i) * LDA + k + qq] : 0.f;
    }
  }
  __syncthreads();

  // ---------------- phase B: the matrix J that Jacobi orthogonalizes -------
  // J = Z when Z is square (p == b); otherwise J = R_Z from a QR of Z.
  float *J = smem;                       // c columns, stride sj
  float *H = smem + lay.j;               // c columns, stride sj
  const float *sig_old = X.sig + (size_t)u * r;
  if (m == c) {
    for (int idx = tid; idx < c * sj; idx += NT) {
      const int col = idx / sj, row = idx - col * sj;
      float v = 0.f;
      if (row < m && col < c) {
        if (row < k)
          v = (row == col) ? sig_old[col] : 0.f;
        else
          v = YFP[(row - k) * D + col];  // col < k: F B ; col >= k: F P
      }
      J[idx] = v;
    }
  } else {
    float *Zb = smem;  // m x c column-major, column stride mz
    const int mz = ldz(m);
    for (int idx = tid; idx < m * c; idx += NT) {
      const int col = idx / m, row = idx - col * m;
      float v;
      if (row < k)
        v = (row == col) ? sig_old[col] : 0.f;
      else
        v = YFP[(row - k) * D + col];
      Zb[(size_t)col * mz + row] = v;
    }
    __syncthreads();
    house_qr<2 * D / 4, false>(Zb, mz, m, c, c, tau);
    // Move R (upper triangle, c x c) into the J layout through registers:
    // the packed upper triangle is dealt evenly over the threads, then the
    // (overlapping) J region is cleared and written.
    constexpr int PER = (D * (D + 1) / 2 + NT - 1) / NT;
    const int ntri = c * (c + 1) / 2;
    float hold[PER];
#pragma unroll
    for (int z = 0; z < PER; z++) {
      const int e = tid + NT * z;
      hold[z] = 0.f;
      if (e < ntri) {
        int col, row;
        tri_index(e, col, row);
        hold[z] = Zb[(size_t)col * mz + row];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < c * sj; idx += NT) J[idx] = 0.f;
    __syncthreads();
#pragma unroll
    for (int z = 0; z < PER; z++) {
      const int e = tid + NT * z;
      if (e < ntri) {
        int col, row;
        tri_index(e, col, row);
        J[(size_t)col * sj + row] = hold[z];
      }
    }
  }
  for (int idx = tid; idx < c * sj; idx += NT) {
    const int col = idx / sj, row = idx - col * sj;
    H[idx] = (row == col) ? 1.f : 0.f;
  }
  __syncthreads();

  // ---------------- phase C: one-sided Jacobi on the columns of J ----------
  {
    float fr = 0.f;
    for (int idx = tid; idx < c * sj; idx += NT) fr += J[idx] * J[idx];
    fr = sum64(fr);
    if ((tid & 63) == 0) sv[tid >> 6] = fr;
    __syncthreads();
    const float fro2 = sv[0] + sv[1] + sv[2] + sv[3];
    // Column dot products are accumulated in fp64 (full rate on this part),
    // so a pair is rotated while its cosine exceeds 8 * 2^-24: just above what
    // rotating fp32 columns can reach, far below the c * 2^-24 a fp32 dot
    // product could resolve. Each fold then leaves its stored coordinates
    // orthogonal to a few fp32 ulps instead of c ulps, which is what keeps
    // hundreds of successive folds on the exact-arithmetic trajectory.
    const double tol = 8.0 * 5.9604644775390625e-8;
    const float ntol = (float)c * 5.9604645e-8f;  // columns below ntol * ||J|| are rounding noise
    const double negl = (double)(ntol * ntol * fro2);
    __syncthreads();  // sv is reused below
    const int c2 = c + (c & 1);
    double *nrm = (double *)tau;  // c squared column norms (tau and sv are free during the sweeps)
    int sweep = 0;
    bool conv = (c < 2);
    // rows per quad lane as a compile-time constant: the loads of a column
    // are then issued back to back
    switch (rl / 4) {
      case 1: jacobi_sweeps<1>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      case 2: jacobi_sweeps<2>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      case 3: jacobi_sweeps<3>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      case 4: jacobi_sweeps<4>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      case 5: jacobi_sweeps<5>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      case 6: jacobi_sweeps<6>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      case 7: jacobi_sweeps<7>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
      default: jacobi_sweeps<8>(J, H, nrm, sj, rl, c, c2, tol, negl, sweep, conv); break;
    }
    if (tid == 0) {
      if (!conv) atomicOr(a.status, FLAG_SWEEP_CAP);
      X.sweeps[u] = sweep;
    }
  }

  // ---------------- phase D: sort, sign, B+, H_top, new rows --------------
  if (tid < k) tau[tid] = sig_old[tid];  // tau is dead after phase B; sigma is rewritten below
  for (int col = qid; col < c; col += NT / 4) {
    const float *zc = J + (size_t)col * sj + q * rl;
    float s = 0.f;
    for (int e = 0; e < rl; e++) s += zc[e] * zc[e];
    s = quad_sum(s);
    if (q == 0) sv[col] = sqrtf(s);
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
  const float sig_jac = (tid < kplus) ? sv[perm[tid]] : 0.f;  // the core's singular value, rank tid
  {
    float *sig_new = X.sig + (size_t)u * r;
    // the old sigma was read only in phase B; safe to overwrite now
    if (tid < r) sig_new[tid] = sig_jac;
    if (tid == 0) {
      float dsum = 0.f;
      for (int qq = kplus; qq < c; qq++) dsum += sv[perm[qq]] * sv[perm[qq]];
      X.disc[u] = dsum;
    }
  }

  // B+ = [B P] H_r into the J region (rows j' x D), 32 rows at a time
  float *Bp = J;
  __syncthreads();  // every thread is done with J before B+ overwrites it
  {
    const int cq = tid & 31;  // columns 4cq .. 4cq+3
    const int rg = tid >> 5;  // rows rg, rg+8, rg+16, rg+24 of each chunk
    for (int j0 = 0; j0 < kplus; j0 += 32) {
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
              const int jr = j0 + rg + 8 * z;
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
        const int jr = j0 + rg + 8 * z;
        if (jr < kplus)
          *reinterpret_cast<float4 *>(Bp + (size_t)jr * D + 4 * cq) = float4{acc[z][0], acc[z][1], acc[z][2], acc[z][3]};
      }
    }
  }
  __syncthreads();
  // sign rule: entry of largest magnitude (lowest index on ties) positive
  for (int jr = grp; jr < kplus; jr += 16) {
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
  // Re-orthonormalization. In exact arithmetic B+ has orthonormal rows and
  // H is orthogonal; in fp32 each fold leaves errors of a few ulps, and B+
  // inherits the previous basis's error, so uncorrected the basis drifts
  // linearly with the number of folds. Two Gram errors are measured:
  //   E   = B+ B+^T - I      (everything: H and the basis [B P])
  //   E_H = H_r^T H_r - I    (the accumulated rotations alone).
  // (I - E/2) B+ is orthonormal to O(E^2). A rotation error inflates C+ = Z H_r
  // and B+ alike, so it is removed from both sides (factor I - E_H/2); a basis
  // error belongs to the coordinates, which take the inverse factor of its
  // share. C+ therefore takes G = I + E/2 - E_H, and sigma its diagonal, so
  // the stored sigma stays the column norms of the stored coordinates.
  // Both matrices live in the fold scratch, which is dead once B+ is formed.
  for (int idx = tid; idx < kplus * D; idx += NT) Bp[idx] *= sgn[idx / D];
  __syncthreads();
  float *Eg = Pg;                             // kplus x kplus: E
  float *Gg = Pg + (size_t)kplus * kplus;     // kplus x kplus: E/2 - E_H
  for (int e = tid; e < kplus * kplus; e += NT) {
    const int i = e / kplus, j = e - i * kplus;
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
    Eg[e] = (float)(acc - dl);
    Gg[e] = (float)(0.5 * (acc - dl) - (ah - dl));
  }
  __syncthreads();
  {
    // B = (I - E/2) B+ straight to the output basis; lanes own columns, so
    // every E entry a wave reads is uniform across it
    const int wv = tid >> 6, ln = tid & 63;
    float *Btw = X.Bt + (size_t)u * r * D;
    for (int i0 = 4 * wv; i0 < kplus; i0 += 16) {
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
    for (int idx = kplus * D + tid; idx < r * D; idx += NT) Btw[idx] = 0.f;
  }
  __syncthreads();  // B+ in the J region is dead from here on
  // Hn = H_r G, signs and rank order applied, column-major (stride sj)
  float *Hn = J;
  {
    const int wv = tid >> 6, ln = tid & 63;
    for (int j0 = 4 * wv; j0 < kplus; j0 += 16) {
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
    for (int idx = tid; idx < k * kplus; idx += NT) {
      const int i = idx / kplus, jr = idx - i * kplus;
      Ht[(size_t)i * r + jr] = Hn[(size_t)jr * sj + i];
    }
  }
  // new rows C[n + i] = [F B | F P]_i Hn (b x k+), staged through the H region
  float *Ys = H;  // b x c, row stride c (b * c <= c * sj)
  for (int idx = tid; idx < b * c; idx += NT) {
    const int i = idx / c, l = idx - i * c;
    Ys[idx] = YFP[(size_t)i * D + l];
  }
  __syncthreads();
  // Each thread owns one column and a strided set of rows, so the squared
  // column norms of the new rows reduce in a fixed order.
  float *part = sv;  // ngrp x r partial sums (sv and sgn are dead here)
  const int ngrp = NT / r;
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
    // With fixed coordinates the stored old rows are not rotated, so their
    // column norms mean nothing: sigma is the core's (times its correction).
    if (a.mode == MODE_FIXED_COORDS)
      X.sig[(size_t)u * r + tid] = (tid < kplus) ? sig_jac * (1.f + Gg[(size_t)tid * kplus + tid]) : 0.f;
    else
      X.sig[(size_t)u * r + tid] = sqrtf(s2);
  }
}

template <int NR, typename TK, typename TC>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) k_core(const FoldArgs a) {
  extern __shared__ float smem[];
  if (blockIdx.y == 0)
    core_body<NR, TK, TC, 0>(a, smem);
  else
    core_body<NR, TK, TC, 1>(a, smem);
}

template <int NR, typename TK, typename TC>
hipError_t launch_core_t(const FoldArgs &a, int nunits, hipStream_t s) {
  size_t lds = core_lds_bytes(a.k[0], a.b, a.r[0]);
  const size_t lv = core_lds_bytes(a.k[1], a.b, a.r[1]);
  if (lv > lds) lds = lv;
  auto kern = k_core<NR, TK, TC>;
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nunits, 2), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <typename TK, typename TC>
hipError_t launch_core_nr(const FoldArgs &a, int nunits, hipStream_t s) {
  const int nr = (a.b + 15) / 16;
  if (nr <= 1) return launch_core_t<1, TK, TC>(a, nunits, s);
  if (nr <= 2) return launch_core_t<2, TK, TC>(a, nunits, s);
  if (nr <= 4) return launch_core_t<4, TK, TC>(a, nunits, s);
  return launch_core_t<8, TK, TC>(a, nunits, s);
}

// ---------------------------------------------------------------------------
// One-shot prefill ([iS-KV] Prefill Compression: the prompt's rows of a unit
// factorised at once by a truncated SVD, k = min(r, rows, d)). The SVD goes
// through the R factor: the rows are taken 128 at a time and folded into R
// by a Householder QR of [R; rows] (R keeps the right singular vectors and
// singular values of all rows seen). Then the columns of R^T (the rows of R)
// are orthogonalised by the same one-sided Jacobi as the fold's core: R^T H
// = V Sigma, so each kept right singular vector is a converged column over
// its norm. Rows of R beyond the rank of the rows are rounding noise and stay
// frozen as negligible columns, so no real content is left behind in them
// (orthogonalising the columns of R instead would freeze shrinking columns
// that still hold content at the threshold's level). The kept vectors,
// signed by the sign rule, become the basis; k_oneshot_coords then stores
// the coordinates C = X B and sigma as their column norms.
// ---------------------------------------------------------------------------
constexpr int OS_M = 2 * D;  // rows of [R; block]

__host__ __device__ inline int oneshot_small() {  // float offset of tau, sv, sgn, perm
  const int z = D * ldz(OS_M);
  const int jh = 2 * D * jac_stride(D);
  return z > jh ? z : jh;
}

// One step of the blockwise QR: [R; X] -> [R'; 0], R upper triangular (D x
// D, rows 0..D-1 of A) and X a block of D rows (rows D..2D-1), column-major
// with column stride ld. Reflector j acts on row j and the block rows only:
// the rows of R below its diagonal are zero and stay zero, so they are never
// touched (half the work of a QR of the full 2D rows). Quad qid owns the
// columns qid, qid + 64; lane q holds block rows D + q + 4e. The owner of
// column j+1 builds reflector j+1 as soon as it has applied reflector j (one
// barrier per reflector); the reflector's block part is kept in column j.
__device__ __forceinline__ void tsqr_step(float *A, int ld, float *tau) {
  constexpr int RQ = D / 4;
  const int tid = threadIdx.x, q = tid & 3, qid = tid >> 2;
  auto reflector = [&](int j) {
    float *cj = A + (size_t)j * ld;
    float x[RQ], sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < RQ; e++) {
      x[e] = cj[D + q + 4 * e];
      sp[e & 3] += x[e] * x[e];
    }
    const float s = quad_sum((sp[0] + sp[1]) + (sp[2] + sp[3]));
    const float x0 = cj[j];
    float tj = 0.f, beta = x0, scal = 0.f;
    if (s > 0.f) {
      beta = -copysignf(sqrtf(x0 * x0 + s), x0);
      tj = (beta - x0) / beta;
      scal = 1.f / (x0 - beta);
    }
#pragma unroll
    for (int e = 0; e < RQ; e++) cj[D + q + 4 * e] = x[e] * scal;
    if (q == 0) {
      cj[j] = beta;
      tau[j] = tj;
    }
  };
  if (qid == 0) reflector(0);
  __syncthreads();
  for (int j = 0; j < D; j++) {
    const float tj = tau[j];
    if (tj != 0.f) {
      const float *cj = A + (size_t)j * ld;
      float v[RQ];
#pragma unroll
      for (int e = 0; e < RQ; e++) v[e] = cj[D + q + 4 * e];
      int col = qid;
      while (col <= j) col += NT / 4;
      for (; col < D; col += NT / 4) {
        float *cc = A + (size_t)col * ld;
        float x[RQ], wp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < RQ; e++) {
          x[e] = cc[D + q + 4 * e];
          wp[e & 3] += v[e] * x[e];
        }
        const float rjc = cc[j];
        const float w = tj * (rjc + quad_sum((wp[0] + wp[1]) + (wp[2] + wp[3])));
#pragma unroll
        for (int e = 0; e < RQ; e++) cc[D + q + 4 * e] = x[e] - w * v[e];
        if (q == 0) cc[j] = rjc - w;
      }
    }
    if (j + 1 < D && qid == ((j + 1) & (NT / 4 - 1))) reflector(j + 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Cholesky-QR of long prompts. The R factor of a unit's rows X (nrows x 128)
// is also the Cholesky factor of G = X^T X, and bf16 or fp32 rows are exact in
// fp64, so G accumulated in fp64 on matrix cores (v_mfma_f64_16x16x4_f64) is
// correct to fp64 rounding; its Cholesky factor then takes 128 steps instead
// of one reflector per row of the blockwise QR. In fp64 the Gram matrix costs
// a singular value sigma_j an absolute error near 1e-16 sigma_1^2 / sigma_j.
// A pivot at or below 1e-13 of G's largest diagonal entry (a column within
// about 3e-7 of the largest column norm of the span of the earlier ones, as in
// rows of lower rank than 128) leaves a zero row of R, which the Jacobi treats
// as negligible, like the QR's rows beyond the rank; dividing by such a pivot
// would magnify the rounding of G instead.
//
// k_oneshot_gram: one workgroup per unit stream (grid (units, 2)). Rows are
// staged 64 at a time in LDS as fp32; the 36 upper-triangle 16 x 16 tiles of
// G are shared out over the 4 waves (9 each, fixed at compile time so the
// operands stay in registers); lane l feeds row r + l / 16, column
// 16 t + l % 16 to both operands (A = X^T tile, B = X tile). G (128 x 128,
// symmetric, fp64) is written to the start of the unit's coordinate region,
// which the coordinates kernel overwrites afterwards.
// ---------------------------------------------------------------------------
constexpr int GCH = 64;      // rows per staged chunk
constexpr int GXS = D + 4;   // staged row stride (floats)

__device__ __forceinline__ double *gram_scratch(const Stream &X, int u, int cb) {
  const uintptr_t p = (uintptr_t)((char *)X.C + (size_t)u * X.cstride * cb);
  return (double *)((p + 7) & ~(uintptr_t)7);
}

typedef __attribute__((ext_vector_type(4))) double g64x4;

// upper-triangle tile e, row-major over ti <= tj
struct GTile {
  int ti, tj;
};
constexpr GTile gram_tile(int e) {
  int tj = 0;
  while ((tj + 1) * (tj + 2) / 2 <= e) tj++;
  return GTile{e - tj * (tj + 1) / 2, tj};
}

template <typename TK, int W>
__device__ __forceinline__ void oneshot_gram_wave(const OneshotArgs &a, const TK *src, float *xs, double *G) {
  constexpr int NTILE = 9;  // 36 tiles / 4 waves
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, lk = lane >> 4;
  g64x4 acc[NTILE];
#pragma unroll
  for (int m = 0; m < NTILE; m++) acc[m] = g64x4{0.0, 0.0, 0.0, 0.0};
  constexpr int PE = 16 / (int)sizeof(TK);  // elements per 16-byte piece
  constexpr int NP = GCH * (D / PE) / NT;   // pieces per thread and chunk
  static_assert(NP * NT == GCH * (D / PE), "whole pieces per thread");
  // the next chunk's pieces are loaded into registers while the matrix cores
  // work on the current one
  uint4 nx[NP];
  auto fetch = [&](int r0) {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      const int idx = tid + NT * p, i = idx / (D / PE), c = idx - i * (D / PE);
      nx[p] = (r0 + i < a.nrows) ? *(const uint4 *)(src + (size_t)(r0 + i) * D + PE * c) : uint4{0, 0, 0, 0};
    }
  };
  fetch(0);
  for (int r0 = 0; r0 < a.nrows; r0 += GCH) {
    __syncthreads();  // the previous chunk is no longer read
#pragma unroll
    for (int p = 0; p < NP; p++) {
      const int idx = tid + NT * p, i = idx / (D / PE), c = idx - i * (D / PE);
      const uint32_t ww[4] = {nx[p].x, nx[p].y, nx[p].z, nx[p].w};
      float v[PE];
      if constexpr (PE == 8) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          v[2 * e] = __uint_as_float(ww[e] << 16);
          v[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = __uint_as_float(ww[e]);
      }
#pragma unroll
      for (int e = 0; e < PE; e++) xs[i * GXS + PE * c + e] = v[e];
    }
    __syncthreads();
    if (r0 + GCH < a.nrows) fetch(r0 + GCH);
    for (int k0 = 0; k0 < GCH; k0 += 4) {
      double x[D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; t++) x[t] = (double)xs[(k0 + lk) * GXS + 16 * t + l16];
#pragma unroll
      for (int m = 0; m < NTILE; m++) {
        const GTile g = gram_tile(W + 4 * m);
        acc[m] = __builtin_amdgcn_mfma_f64_16x16x4f64(x[g.ti], x[g.tj], acc[m], 0, 0, 0);
      }
    }
  }
  // element v of lane l: G[16 ti + l / 16 + 4 v][16 tj + l % 16], mirrored
#pragma unroll
  for (int m = 0; m < NTILE; m++) {
    const GTile g = gram_tile(W + 4 * m);
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int i = 16 * g.ti + lk + 4 * v, j = 16 * g.tj + l16;
      G[(size_t)i * D + j] = acc[m][v];
      G[(size_t)j * D + i] = acc[m][v];
    }
  }
}

template <typename TK>
__global__ void __launch_bounds__(NT) k_oneshot_gram(const OneshotArgs a) {
  __shared__ float xs[GCH * GXS];
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int lrel = ul / (a.batch * a.kvh), rem = ul - lrel * (a.batch * a.kvh);
  const int bi = rem / a.kvh, hh = rem - bi * a.kvh;
  const int xk = blockIdx.y, wv = threadIdx.x >> 6;
  const TK *src = (const TK *)a.src[xk] + (((size_t)bi * a.nl_in + a.lrel0 + lrel) * a.kvh + hh) * (size_t)a.nrows * D;
  double *G = gram_scratch(a.X[xk], u, a.cb);
  switch (wv) {
    case 0: oneshot_gram_wave<TK, 0>(a, src, xs, G); break;
    case 1: oneshot_gram_wave<TK, 1>(a, src, xs, G); break;
    case 2: oneshot_gram_wave<TK, 2>(a, src, xs, G); break;
    default: oneshot_gram_wave<TK, 3>(a, src, xs, G); break;
  }
}

// Cholesky G = R^T R in LDS (fp64, R upper triangular in place, row j of R in
// row j of Gs); a pivot at or below 1e-13 of the largest diagonal entry leaves
// row j zero
__device__ __forceinline__ void gram_cholesky(double *Gs) {
  const int tid = threadIdx.x;
  double gmax = 0.0;
  for (int j = 0; j < D; j++) gmax = fmax(gmax, Gs[(size_t)j * D + j]);
  const double tol = 1e-13 * gmax;
  for (int j = 0; j < D; j++) {
    const double d = Gs[(size_t)j * D + j];
    const double rjj = d > tol ? sqrt(d) : 0.0;
    const double inv = rjj > 0.0 ? 1.0 / rjj : 0.0;
    __syncthreads();  // every thread has read the pivot before row j changes
    if (tid >= j && tid < D) Gs[(size_t)j * D + tid] = (tid == j) ? rjj : Gs[(size_t)j * D + tid] * inv;
    __syncthreads();
    const int m = D - 1 - j;
    for (int idx = tid; idx < m * m; idx += NT) {
      const int i = j + 1 + idx / m, k = j + 1 + idx % m;
      if (i <= k) Gs[(size_t)i * D + k] -= Gs[(size_t)j * D + i] * Gs[(size_t)j * D + k];
    }
    __syncthreads();
  }
}

template <typename TK, int XK>
__device__ void oneshot_svd_body(const OneshotArgs &a, float *smem) {
  const Stream &X = a.X[XK];
  const int tid = threadIdx.x, q = tid & 3, qid = tid >> 2, lane = tid & 63, wv = tid >> 6;
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int lrel = ul / (a.batch * a.kvh), rem = ul - lrel * (a.batch * a.kvh);
  const int bi = rem / a.kvh, hh = rem - bi * a.kvh;
  const TK *src = (const TK *)a.src[XK] +
                  (((size_t)bi * a.nl_in + a.lrel0 + lrel) * a.kvh + hh) * (size_t)a.nrows * D;
  const int r = X.r;
  const int kplus = min(min(r, a.nrows), D);
  float *tau = smem + oneshot_small();
  float *sv = tau + D;
  float *sgn = sv + D;
  int *perm = (int *)(sgn + D);
  float *Zb = smem;
  const int mz = ldz(OS_M);
  if (a.gram) {
    // G into LDS (fp64, 128 x 128 over the QR's region), R by Cholesky, R in
    // fp32 through global memory behind G, then into R's place in Zb
    double *G = gram_scratch(X, u, a.cb);
    float *Rg = (float *)(G + D * D);
    double *Gs = (double *)smem;
    for (int idx = tid; idx < D * D; idx += NT) Gs[idx] = G[idx];
    __syncthreads();
    gram_cholesky(Gs);
    for (int idx = tid; idx < D * D; idx += NT) {
      const int row = idx / D, col = idx - row * D;
      Rg[idx] = row <= col ? (float)Gs[idx] : 0.f;
    }
    __threadfence();
    __syncthreads();
    for (int idx = tid; idx < D * D; idx += NT) {
      const int col = idx / D, row = idx - col * D;
      Zb[(size_t)col * mz + row] = Rg[(size_t)row * D + col];
    }
    __syncthreads();
    // the scratch lies in the coordinate region, rows past the prompt included:
    // clear it rather than leave fp64 bit patterns there
    for (int idx = tid; idx < D * D * 3 / 2; idx += NT) G[idx] = 0.0;
  } else {
  for (int idx = tid; idx < D * mz; idx += NT) Zb[idx] = 0.f;
  __syncthreads();
  for (int r0 = 0; r0 < a.nrows; r0 += D) {
    // rows r0 .. r0+127 below R (zero past the last row)
    for (int idx = tid; idx < D * D; idx += NT) {
      const int i = idx / D, t = idx - i * D;
      Zb[(size_t)t * mz + D + i] = (r0 + i < a.nrows) ? ldf<TK>(src, (size_t)(r0 + i) * D + t) : 0.f;
    }
    __syncthreads();
    tsqr_step(Zb, mz, tau);  // R's rows below its diagonal stay zero; the block rows are reloaded
  }
  }
  // R^T (R's rows as columns) into the Jacobi layout through registers, H = I
  const int c = D, sj = jac_stride(D), rl = jac_rl(D);
  float *J = smem, *H = smem + c * sj;
  {
    constexpr int PER = (D * (D + 1) / 2 + NT - 1) / NT;
    const int ntri = D * (D + 1) / 2;
    float hold[PER];
#pragma unroll
    for (int z = 0; z < PER; z++) {
      const int e = tid + NT * z;
      hold[z] = 0.f;
      if (e < ntri) {
        int col, row;
        tri_index(e, col, row);
        hold[z] = Zb[(size_t)col * mz + row];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < c * sj; idx += NT) {
      const int col = idx / sj, row = idx - col * sj;
      J[idx] = 0.f;
      H[idx] = (row == col) ? 1.f : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int z = 0; z < PER; z++) {
      const int e = tid + NT * z;
      if (e < ntri) {
        int col, row;
        tri_index(e, col, row);
        J[(size_t)row * sj + col] = hold[z];
      }
    }
    __syncthreads();
  }
  double negl;
  {
    float fr = 0.f;
    for (int idx = tid; idx < c * sj; idx += NT) fr += J[idx] * J[idx];
    fr = sum64(fr);
    if (lane == 0) sv[wv] = fr;
    __syncthreads();
    const float fro2 = sv[0] + sv[1] + sv[2] + sv[3];
    const double tol = 8.0 * 5.9604644775390625e-8;
    const float ntol = (float)c * 5.9604645e-8f;
    negl = (double)(ntol * ntol * fro2);
    __syncthreads();
    double *nrm = (double *)tau;
    int sweep = 0;
    bool conv = false;
    jacobi_sweeps<D / 16>(J, H, nrm, sj, rl, c, c, tol, negl, sweep, conv);
    if (tid == 0) {
      if (!conv) atomicOr(a.status, FLAG_SWEEP_CAP);
      X.sweeps[u] = sweep;
    }
  }
  // singular values, rank order (non-finite ones flagged and ranked last)
  for (int col = qid; col < c; col += NT / 4) {
    const float *zc = J + (size_t)col * sj + q * rl;
    float s = 0.f;
    for (int e = 0; e < rl; e++) s += zc[e] * zc[e];
    s = quad_sum(s);
    if (q == 0) {
      float v = sqrtf(s);
      if (!(v <= 3.0e38f)) {
        atomicOr(a.status, FLAG_NONFINITE);
        v = -1.f;
      }
      sv[col] = v;
    }
  }
  __syncthreads();
  if (tid < c) {
    const float me = sv[tid];
    int rank = 0;
    for (int i = 0; i < c; i++) {
      const float o = sv[i];
      rank += (o > me || (o == me && i < tid)) ? 1 : 0;
    }
    perm[rank] = tid;
  }
  __syncthreads();
  // basis rows, staged in the H region (free now): converged column perm[jr]
  // over its norm; a kept column at the rounding level (rows of rank below k)
  // is completed instead by the first unit vector e_t that keeps a norm above
  // 1/2 after two Gram-Schmidt passes against the rows before it
  float *Bs = H;  // r x D
  const float neglf = (float)negl;
  for (int idx = tid; idx < kplus * D; idx += NT) {
    const int jr = idx / D, t = idx - jr * D;
    const int col = perm[jr];
    const float sc = sv[col];
    Bs[idx] = (sc * sc > neglf) ? J[(size_t)col * sj + t] / sc : 0.f;
  }
  __syncthreads();
  if (wv == 0) {
    int t_next = 0;
    for (int jr = 0; jr < kplus; jr++) {
      const float sc = sv[perm[jr]];
      if (sc * sc > neglf) continue;
      for (; t_next < D; t_next++) {
        float w0 = (lane == t_next) ? 1.f : 0.f, w1 = (lane + 64 == t_next) ? 1.f : 0.f;
        for (int pass = 0; pass < 2; pass++) {
          for (int i = 0; i < kplus; i++) {
            if (i == jr) continue;
            const float b0 = Bs[(size_t)i * D + lane], b1 = Bs[(size_t)i * D + lane + 64];
            const float pr = sum64(w0 * b0 + w1 * b1);
            w0 -= pr * b0;
            w1 -= pr * b1;
          }
        }
        const float nn = sqrtf(sum64(w0 * w0 + w1 * w1));
        if (nn > 0.5f) {
          Bs[(size_t)jr * D + lane] = w0 / nn;
          Bs[(size_t)jr * D + lane + 64] = w1 / nn;
          t_next++;
          break;
        }
      }
    }
  }
  __syncthreads();
  // sign rule: the entry of largest magnitude (lowest index on ties) of each
  // basis vector is positive; one wave per row
  float *Btw = X.Bt + (size_t)u * r * D;
  for (int jr = wv; jr < r; jr += NT / 64) {
    if (jr < kplus) {
      const float h0 = Bs[(size_t)jr * D + lane], h1 = Bs[(size_t)jr * D + lane + 64];
      float best = fabsf(h0);
      int bi2 = lane;
      if (fabsf(h1) > best) {
        best = fabsf(h1);
        bi2 = lane + 64;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi2, off);
        if (ob > best || (ob == best && oi < bi2)) {
          best = ob;
          bi2 = oi;
        }
      }
      const float sg = (Bs[(size_t)jr * D + bi2] < 0.f) ? -1.f : 1.f;
      Btw[(size_t)jr * D + lane] = sg * h0;
      Btw[(size_t)jr * D + lane + 64] = sg * h1;
    } else {
      Btw[(size_t)jr * D + lane] = 0.f;
      Btw[(size_t)jr * D + lane + 64] = 0.f;
    }
  }
  if (tid == 0) {
    float dsum = 0.f;
    for (int i = kplus; i < c; i++) dsum += sv[perm[i]] * sv[perm[i]];
    X.disc[u] = dsum;
  }
}

// one workgroup per CU (its LDS is 136 KB), so each wave may take the whole
// register file
template <typename TK>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) k_oneshot_svd(const OneshotArgs a) {
  extern __shared__ float smem[];
  if (blockIdx.y == 0)
    oneshot_svd_body<TK, 0>(a, smem);
  else
    oneshot_svd_body<TK, 1>(a, smem);
}

// rows staged per pass of k_oneshot_coords: one thread per (row, column),
// at most 64 rows (keeps the LDS of small ranks bounded)
__host__ __device__ inline int oneshot_rows_per_pass(int r) { return NT / r < 64 ? NT / r : 64; }

// C[i] = X_i B (kplus columns, zero to r) for every prompt row; sigma = the
// column norms of the coordinates as stored. Rows are staged in LDS NT / r at
// a time; thread (g, j) owns column j of row g of each pass.
template <typename TK, typename TC>
__global__ void __launch_bounds__(NT) k_oneshot_coords(const OneshotArgs a) {
  extern __shared__ float smem[];
  const int XK = blockIdx.y;
  const Stream &X = a.X[XK];
  const int tid = threadIdx.x;
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int lrel = ul / (a.batch * a.kvh), rem = ul - lrel * (a.batch * a.kvh);
  const int bi = rem / a.kvh, hh = rem - bi * a.kvh;
  const TK *src = (const TK *)a.src[XK] +
                  (((size_t)bi * a.nl_in + a.lrel0 + lrel) * a.kvh + hh) * (size_t)a.nrows * D;
  const int r = X.r;
  const int kplus = min(min(r, a.nrows), D);
  const int G = oneshot_rows_per_pass(r);  // rows per pass
  float *Bs = smem;                      // r x (D + 1)
  float *xs = Bs + (size_t)r * (D + 1);  // G x D
  float *part = xs + (size_t)G * D;      // G x r
  const float *Bt = X.Bt + (size_t)u * r * D;
  for (int idx = tid; idx < r * D; idx += NT) {
    const int j = idx / D, t = idx - j * D;
    Bs[j * (D + 1) + t] = Bt[idx];
  }
  TC *Cu = (TC *)X.C + (size_t)u * X.cstride;
  const int g0 = tid / r, j = tid - g0 * r;
  float sq = 0.f;
  for (int i0 = 0; i0 < a.nrows; i0 += G) {
    __syncthreads();  // xs free (and Bs written, first pass)
    for (int idx = tid; idx < G * D; idx += NT) {
      const int g = idx / D, t = idx - g * D;
      xs[idx] = (i0 + g < a.nrows) ? ldf<TK>(src, (size_t)(i0 + g) * D + t) : 0.f;
    }
    __syncthreads();
    const int i = i0 + g0;
    if (g0 < G && i < a.nrows) {
      float s = 0.f;
      if (j < kplus) {
        const float *xr = xs + (size_t)g0 * D, *br = Bs + (size_t)j * (D + 1);
#pragma unroll 8
        for (int t = 0; t < D; t++) s += xr[t] * br[t];
      }
      stf<TC>(Cu, (size_t)i * r + j, s);
      const float st = ldf<TC>(Cu, (size_t)i * r + j);
      sq += st * st;
    }
  }
  __syncthreads();
  if (g0 < G) part[g0 * r + j] = sq;
  __syncthreads();
  if (tid < r) {
    float s2 = 0.f;
    for (int g = 0; g < G; g++) s2 += part[g * r + tid];
    X.sig[(size_t)u * r + tid] = (tid < kplus) ? sqrtf(s2) : 0.f;
  }
}

}  // namespace

size_t core_lds_bytes(int k, int b, int r) {
  return sizeof(float) * ((size_t)core_lds(k, b, r).total + 4 * D);
}

hipError_t launch_core(const FoldArgs &a0, int nunits, int kv_bf16, int coord_bf16, hipStream_t s) {
  FoldArgs a = a0;
  for (int x = 0; x < 2; x++) a.lds_small[x] = core_lds(a.k[x], a.b, a.r[x]).total;
  if (kv_bf16 && coord_bf16) return launch_core_nr<uint16_t, uint16_t>(a, nunits, s);
  if (kv_bf16 && !coord_bf16) return launch_core_nr<uint16_t, float>(a, nunits, s);
  if (!kv_bf16 && coord_bf16) return launch_core_nr<float, uint16_t>(a, nunits, s);
  return launch_core_nr<float, float>(a, nunits, s);
}

hipError_t launch_oneshot(const OneshotArgs &a0, int nunits, int kv_bf16, int coord_bf16, hipStream_t s) {
  const size_t lds1 = sizeof(float) * ((size_t)oneshot_small() + 4 * D);
  hipError_t e;
  // long prompts: R from the Cholesky factor of the fp64 Gram matrix, which
  // (with R in fp32 behind it) is kept in the units' coordinate regions, when
  // they can hold it, and read from 16-byte aligned rows
  OneshotArgs a = a0;
  a.cb = a.X[0].cs ? 1 : coord_bf16 ? 2 : 4;
  const size_t need = (size_t)D * D * (sizeof(double) + sizeof(float)) + 8;
  a.gram = a.nrows >= 1024 && (((uintptr_t)a.src[0] | (uintptr_t)a.src[1]) & 15) == 0 &&
           a.X[0].cstride * a.cb >= need && a.X[1].cstride * a.cb >= need;
  if (a.gram) {
    if (kv_bf16)
      hipLaunchKernelGGL(k_oneshot_gram<uint16_t>, dim3(nunits, 2), dim3(NT), 0, s, a);
    else
      hipLaunchKernelGGL(k_oneshot_gram<float>, dim3(nunits, 2), dim3(NT), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (kv_bf16) {
    e = hipFuncSetAttribute((const void *)k_oneshot_svd<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_oneshot_svd<uint16_t>, dim3(nunits, 2), dim3(NT), lds1, s, a);
  } else {
    e = hipFuncSetAttribute((const void *)k_oneshot_svd<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_oneshot_svd<float>, dim3(nunits, 2), dim3(NT), lds1, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.X[0].cs) return launch_oneshot_coords_i8(a, nunits, s);  // int8 storage of U (bf16 rows)
  if (oneshot_coords_mfma_ok(a, kv_bf16, coord_bf16)) return launch_oneshot_coords_mfma(a, nunits, s);
  const int rmin = a.X[0].r < a.X[1].r ? a.X[0].r : a.X[1].r;
  const int rmax = a.X[0].r > a.X[1].r ? a.X[0].r : a.X[1].r;
  const size_t lds2 = sizeof(float) * ((size_t)rmax * (D + 1) + (size_t)oneshot_rows_per_pass(rmin) * D + NT);
  auto go = [&](const void *kf, auto kern) {
    hipError_t e2 = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL(kern, dim3(nunits, 2), dim3(NT), lds2, s, a);
    return hipGetLastError();
  };
  if (kv_bf16 && coord_bf16) return go((const void *)k_oneshot_coords<uint16_t, uint16_t>, k_oneshot_coords<uint16_t, uint16_t>);
  if (kv_bf16) return go((const void *)k_oneshot_coords<uint16_t, float>, k_oneshot_coords<uint16_t, float>);
  if (coord_bf16) return go((const void *)k_oneshot_coords<float, uint16_t>, k_oneshot_coords<float, uint16_t>);
  return go((const void *)k_oneshot_coords<float, float>, k_oneshot_coords<float, float>);
}

}  // namespace iskv
