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
// Lane groups of 16 lanes do the vector work: a group owns a column (or a
// row) of 128 / 16 = 8 contiguous elements per lane and reduces with xor
// shuffles inside the group.
#include "iskv_internal.hpp"

namespace iskv {

namespace {

// LDS float counts of each phase (see the kernel body)
__host__ __device__ inline int core_phase_floats(int k, int b, int r) {
  const int p = (b < D - k) ? b : D - k;
  const int m = k + b, c = k + p;
  const int sj = 16 * ((c + 15) / 16);
  int a = (k + b + p) * D;              // phase A: [B; E] rows + P accumulation
  int z = (m > c) ? m * c : 0;          // phase B: Z before its QR
  int j = c * D + c * sj;               // phase C/D: J (or B+, or [FB FP]) + H
  int mx = a > z ? a : z;
  return mx > j ? mx : j;
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

// Householder QR (LAPACK dlarfg convention: H = I - tau v v^T, v[0] = 1,
// H x = beta e_0) of an nrows x ncols matrix stored column-major in LDS with
// column stride ld; nref reflectors. On return the upper triangle holds R,
// the part below the diagonal holds v (without the unit head), tau[j] the
// scalars. Rows of a column are split over the 16 lanes of a group with a
// stride of 16. All 256 threads must call it.
__device__ void house_qr(float *A, int ld, int nrows, int ncols, int nref, float *tau) {
  const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4;
  for (int j = 0; j < nref; j++) {
    float *cj = A + (size_t)j * ld;
    if (tid < 64) {
      float s = 0.f;
      for (int t = j + 1 + tid; t < nrows; t += 64) s += cj[t] * cj[t];
      s = sum64(s);
      const float x0 = cj[j];
      float tj = 0.f, beta = x0, scal = 0.f;
      if (s > 0.f) {
        beta = -copysignf(sqrtf(x0 * x0 + s), x0);
        tj = (beta - x0) / beta;
        scal = 1.f / (x0 - beta);
      }
      for (int t = j + 1 + tid; t < nrows; t += 64) cj[t] *= scal;
      __builtin_amdgcn_wave_barrier();
      if (tid == 0) {
        cj[j] = beta;
        tau[j] = tj;
      }
    }
    __syncthreads();
    const float tj = tau[j];
    if (tj != 0.f) {
      for (int col = j + 1 + grp; col < ncols; col += 16) {
        float *cc = A + (size_t)col * ld;
        float part = 0.f;
        for (int t = j + 1 + lane; t < nrows; t += 16) part += cj[t] * cc[t];
        part = sum16(part);
        const float w = tj * (cc[j] + part);
        for (int t = j + 1 + lane; t < nrows; t += 16) cc[t] -= w * cj[t];
        if (lane == 0) cc[j] -= w;
      }
    }
    __syncthreads();
  }
}

template <int NR, typename TK, typename TC>
__global__ void __launch_bounds__(NT) k_core(const FoldArgs a) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4;
  const int u = a.u0 + blockIdx.x;
  const int b = a.b, k = a.k, r = a.r;
  const int p = (b < D - k) ? b : D - k;
  const int m = k + b, c = k + p;
  const int kplus = (r < c) ? r : c;
  const int nj = (c + 15) / 16;  // J/H elements per lane per column
  const int sj = 16 * nj;        // column stride of J and H

  float *tau = smem + a.lds_small;
  float *sv = tau + D;
  float *sgn = sv + D;
  int *perm = (int *)(sgn + D);
  int *misc = perm + D;

  const float *Bt = a.X.Bt + (size_t)u * r * D;
  float *Pg = a.X.P + (size_t)u * a.pmax * D;
  float *YFP = a.X.YFP + (size_t)u * a.bmax * D;
  const TK *ring = (const TK *)a.X.ring + (size_t)u * a.rcap * D;

  // ---------------- phase A: projection, residual, residual basis ---------
  float *A = smem;  // rows 0..k-1 = basis vectors, rows k..k+b-1 = residual rows
  for (int idx = tid; idx < k * D; idx += NT) A[idx] = Bt[idx];
  float f[NR][8];
#pragma unroll
  for (int q = 0; q < NR; q++) {
    const int i = grp + 16 * q;
    if (i < b) {
      int ri = a.head + i;
      if (ri >= a.rcap) ri -= a.rcap;
#pragma unroll
      for (int t = 0; t < 8; t++) f[q][t] = ldf<TK>(ring, (size_t)ri * D + lane * 8 + t);
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++) f[q][t] = 0.f;
    }
  }
  __syncthreads();
  // Y = F B, E = F - Y B^T; then once more against B (E <- E - (E B) B^T, Y += E B)
  for (int pass = 0; pass < 2; pass++) {
    for (int j = 0; j < k; j++) {
      float bj[8];
#pragma unroll
      for (int t = 0; t < 8; t++) bj[t] = A[j * D + lane * 8 + t];
#pragma unroll
      for (int q = 0; q < NR; q++) {
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < 8; t++) s += f[q][t] * bj[t];
        s = sum16(s);
#pragma unroll
        for (int t = 0; t < 8; t++) f[q][t] -= s * bj[t];
        const int i = grp + 16 * q;
        if (lane == 0 && i < b) {
          if (pass == 0)
            YFP[i * D + j] = s;
          else
            YFP[i * D + j] += s;
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NR; q++) {
    const int i = grp + 16 * q;
    if (i < b) {
#pragma unroll
      for (int t = 0; t < 8; t++) A[(k + i) * D + lane * 8 + t] = f[q][t];
    }
  }
  __syncthreads();

  if (p > 0) {
    // Householder QR of [B | E^T] (column j = LDS row j), c reflectors.
    house_qr(A, D, D, k + b, c, tau);
    // P = Q[:, k:k+p] = H_0 ... H_{c-1} [e_k .. e_{k+p-1}], accumulated backwards.
    // Column q lives in the registers of one lane group (row t = lane + 16e),
    // so no LDS traffic or barrier is needed between reflectors. Reflectors
    // j > k+q leave e_{k+q} unchanged and are skipped.
    float *X = A + (size_t)(k + b) * D;
    for (int q = grp; q < p; q += 16) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = (lane + 16 * e == k + q) ? 1.f : 0.f;
      for (int j = k + q; j >= 0; j--) {
        const float tj = tau[j];
        if (tj == 0.f) continue;
        const float *cj = A + (size_t)j * D;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int t = lane + 16 * e;
          part += (t > j) ? cj[t] * x[e] : ((t == j) ? x[e] : 0.f);
        }
        const float w = tj * sum16(part);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int t = lane + 16 * e;
          x[e] -= (t > j) ? w * cj[t] : ((t == j) ? w : 0.f);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; e++) X[(size_t)q * D + lane + 16 * e] = x[e];
    }
    __syncthreads();
    for (int idx = tid; idx < p * D; idx += NT) Pg[idx] = X[idx];
    // F P = R[k:k+p, k:k+b]^T (lower trapezoidal)
    for (int idx = tid; idx < b * p; idx += NT) {
      const int i = idx / p, q = idx - i * p;
      YFP[i * D + k + q] = (q <= i) ? A[(size_t)(k + i) * D + k + q] : 0.f;
    }
  }
  __syncthreads();

  // ---------------- phase B: the matrix J that Jacobi orthogonalizes -------
  // J = Z when Z is square (p == b); otherwise J = R_Z from a QR of Z.
  float *J = smem;                      // c columns, stride sj (region c*D floats)
  float *H = smem + (size_t)c * D;      // c columns, stride sj
  const float *sig_old = a.X.sig + (size_t)u * r;
  if (m == c) {
    for (int idx = tid; idx < c * sj; idx += NT) {
      const int col = idx / sj, row = idx - col * sj;
      float v = 0.f;
      if (row < m) {
        if (row < k)
          v = (row == col) ? sig_old[col] : 0.f;
        else
          v = YFP[(row - k) * D + col];  // col < k: F B ; col >= k: F P
      }
      J[idx] = v;
    }
  } else {
    float *Zb = smem;  // m x c column-major
    for (int idx = tid; idx < m * c; idx += NT) {
      const int col = idx / m, row = idx - col * m;
      float v;
      if (row < k)
        v = (row == col) ? sig_old[col] : 0.f;
      else
        v = YFP[(row - k) * D + col];
      Zb[idx] = v;
    }
    __syncthreads();
    house_qr(Zb, m, m, c, c, tau);
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
        hold[z] = Zb[(size_t)col * m + row];
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
    const float tol = (float)c * 5.9604645e-8f;  // c * 2^-24
    const float negl = tol * tol * fro2;
    __syncthreads();  // sv is reused below
    const int c2 = c + (c & 1);
    int sweep = 0;
    bool conv = (c < 2);
    while (!conv && sweep < SWEEP_CAP) {
      sweep++;
      int rot = 0;
      for (int rnd = 0; rnd < c2 - 1; rnd++) {
        for (int pr = grp; pr < c2 / 2; pr += 16) {
          int ci, cj;
          rr_pair(rnd, pr, c2, ci, cj);
          if (cj >= c) continue;
          float *zi = J + (size_t)ci * sj + lane * nj;
          float *zj = J + (size_t)cj * sj + lane * nj;
          float xi[8], xj[8];
          float al = 0.f, be = 0.f, ga = 0.f;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            if (e < nj) {
              xi[e] = zi[e];
              xj[e] = zj[e];
              al += xi[e] * xi[e];
              be += xj[e] * xj[e];
              ga += xi[e] * xj[e];
            }
          }
          al = sum16(al);
          be = sum16(be);
          ga = sum16(ga);
          if (al > negl && be > negl && fabsf(ga) > tol * sqrtf(al * be)) {
            const float zeta = (be - al) / (2.f * ga);
            const float az = fabsf(zeta);
            float t = (az > 1e18f) ? 0.5f / az : 1.f / (az + sqrtf(1.f + az * az));
            t = copysignf(t, zeta);
            const float cs = 1.f / sqrtf(1.f + t * t);
            const float sn = cs * t;
#pragma unroll
            for (int e = 0; e < 8; e++) {
              if (e < nj) {
                zi[e] = cs * xi[e] - sn * xj[e];
                zj[e] = sn * xi[e] + cs * xj[e];
              }
            }
            float *hi = H + (size_t)ci * sj + lane * nj;
            float *hj = H + (size_t)cj * sj + lane * nj;
#pragma unroll
            for (int e = 0; e < 8; e++) {
              if (e < nj) {
                const float p0 = hi[e], p1 = hj[e];
                hi[e] = cs * p0 - sn * p1;
                hj[e] = sn * p0 + cs * p1;
              }
            }
            rot = 1;
          }
        }
        __syncthreads();
      }
      conv = !__syncthreads_or(rot);
    }
    if (tid == 0) {
      if (!conv) atomicOr(a.status, FLAG_SWEEP_CAP);
      a.X.sweeps[u] = sweep;
    }
  }

  // ---------------- phase D: sort, sign, B+, H_top, new rows --------------
  for (int col = grp; col < c; col += 16) {
    const float *zc = J + (size_t)col * sj + lane * nj;
    float s = 0.f;
    for (int e = 0; e < nj; e++) s += zc[e] * zc[e];
    s = sum16(s);
    if (lane == 0) sv[col] = sqrtf(s);
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
  {
    float *sig_new = a.X.sig + (size_t)u * r;
    // every thread reads the old sigma only in phase B; safe to overwrite now
    if (tid < r) sig_new[tid] = (tid < kplus) ? sv[perm[tid]] : 0.f;
    if (tid == 0) {
      float dsum = 0.f;
      for (int q = kplus; q < c; q++) dsum += sv[perm[q]] * sv[perm[q]];
      a.X.disc[u] = dsum;
    }
  }

  // B+ = [B P] H_r into the J region (rows j' x D)
  __syncthreads();
  float *Bp = J;
  {
    const int cq = tid & 31;  // columns 4cq .. 4cq+3
    const int rg = tid >> 5;  // rows rg, rg+8, ...
    constexpr int ZR = D / 8;
    float acc[ZR][4];
#pragma unroll
    for (int z = 0; z < ZR; z++)
#pragma unroll
      for (int t = 0; t < 4; t++) acc[z][t] = 0.f;
    for (int i = 0; i < c; i++) {
      const float *src = (i < k) ? (Bt + (size_t)i * D) : (Pg + (size_t)(i - k) * D);
      const float4 bp = *reinterpret_cast<const float4 *>(src + 4 * cq);
#pragma unroll
      for (int z = 0; z < ZR; z++) {
        const int jr = rg + 8 * z;
        if (jr < kplus) {
          const float hv = H[(size_t)perm[jr] * sj + i];
          acc[z][0] += hv * bp.x;
          acc[z][1] += hv * bp.y;
          acc[z][2] += hv * bp.z;
          acc[z][3] += hv * bp.w;
        }
      }
    }
#pragma unroll
    for (int z = 0; z < ZR; z++) {
      const int jr = rg + 8 * z;
      if (jr < kplus) {
#pragma unroll
        for (int t = 0; t < 4; t++) Bp[(size_t)jr * D + 4 * cq + t] = acc[z][t];
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
  {
    float *Btw = a.X.Bt + (size_t)u * r * D;
    for (int idx = tid; idx < r * D; idx += NT) {
      const int jr = idx / D;
      Btw[idx] = (jr < kplus) ? sgn[jr] * Bp[idx] : 0.f;
    }
    float *Ht = a.X.Htop + (size_t)u * r * r;
    for (int idx = tid; idx < k * kplus; idx += NT) {
      const int i = idx / kplus, jr = idx - i * kplus;
      Ht[(size_t)i * r + jr] = sgn[jr] * H[(size_t)perm[jr] * sj + i];
    }
  }
  __syncthreads();
  // new rows C[n + i] = [F B | F P]_i H_r (b x k+), staged through LDS
  float *Ys = J;  // b x c, row stride c
  for (int idx = tid; idx < b * c; idx += NT) {
    const int i = idx / c, l = idx - i * c;
    Ys[idx] = YFP[(size_t)i * D + l];
  }
  __syncthreads();
  {
    TC *Cn = (TC *)a.X.C + ((size_t)u * a.ncap + a.n) * r;
    for (int idx = tid; idx < b * r; idx += NT) {
      const int i = idx / r, jr = idx - i * r;
      float s = 0.f;
      if (jr < kplus) {
        const float *hc = H + (size_t)perm[jr] * sj;
        const float *yr = Ys + (size_t)i * c;
        for (int l = 0; l < c; l++) s += yr[l] * hc[l];
        s *= sgn[jr];
      }
      stf<TC>(Cn, (size_t)i * r + jr, s);
    }
  }
}

template <int NR, typename TK, typename TC>
hipError_t launch_core_t(const FoldArgs &a, int nunits, hipStream_t s) {
  const size_t lds = core_lds_bytes(a.k, a.b, a.r);
  auto kern = k_core<NR, TK, TC>;
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nunits), dim3(NT), lds, s, a);
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

}  // namespace

size_t core_lds_bytes(int k, int b, int r) {
  (void)r;
  return sizeof(float) * ((size_t)core_phase_floats(k, b, r) + 4 * D + 8);
}

hipError_t launch_core(const FoldArgs &a0, int nunits, int kv_bf16, int coord_bf16, hipStream_t s) {
  FoldArgs a = a0;
  a.lds_small = core_phase_floats(a.k, a.b, a.r);
  if (kv_bf16 && coord_bf16) return launch_core_nr<uint16_t, uint16_t>(a, nunits, s);
  if (kv_bf16 && !coord_bf16) return launch_core_nr<uint16_t, float>(a, nunits, s);
  if (!kv_bf16 && coord_bf16) return launch_core_nr<float, uint16_t>(a, nunits, s);
  return launch_core_nr<float, float>(a, nunits, s);
}

}  // namespace iskv
