// Device building blocks shared by the fold cores and the one-shot prefill:
// LDS layouts, round-robin pair order, DPP lane-group sums, Householder QR
// of an LDS-resident matrix, and one-sided Jacobi sweeps.
//
// Lane groups: a "quad" is 4 consecutive lanes, an "octet" 8. A quad or
// octet owns one column (QR) or one Jacobi pair; its lanes split the rows in
// contiguous chunks, and their partial sums are combined with DPP moves that
// stay inside the group (no LDS traffic).
#pragma once

#include "iskv_internal.hpp"

namespace iskv {
namespace fold {

constexpr int LDA = D + 4;  // LDS stride of 128-long rows (4 mod 32)
__host__ __device__ inline int ldz(int m) { return ((m + 31) / 32) * 32 + 4; }

// (column, row) of entry e of a column-major packed upper triangle
__device__ __forceinline__ void tri_index(int e, int &col, int &row) {
  int cc = (int)((sqrtf(8.f * (float)e + 1.f) - 1.f) * 0.5f);
  while (cc > 0 && cc * (cc + 1) / 2 > e) cc--;
  while ((cc + 1) * (cc + 2) / 2 <= e) cc++;
  col = cc;
  row = e - cc * (cc + 1) / 2;
}

// pair (i < j) of round `rnd` in a round-robin over c2 players (c2 even):
// every pair meets exactly once in c2 - 1 rounds
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

// DPP move of a double (two 32-bit moves with the same control)
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const int lo = (int)(u & 0xffffffffull), hi = (int)(u >> 32);
  const int lo2 = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false);
  const int hi2 = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi2 << 32) | (unsigned)lo2);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <-> 7 - i within each 8 lanes

// Sum over the 4 lanes of a quad / the 8 lanes of an octet. Every lane ends
// with the same value: a + b is computed as the same two operands on each.
__device__ __forceinline__ double quad_sum_d(double v) {
  v += dpp_d<DPP_QUAD_XOR1>(v);
  v += dpp_d<DPP_QUAD_XOR2>(v);
  return v;
}
__device__ __forceinline__ double octet_sum_d(double v) {
  v = quad_sum_d(v);
  // each lane of one quad meets a lane of the other quad of the octet
  return v + dpp_d<DPP_ROW_HALF_MIRROR>(v);
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), DPP_QUAD_XOR1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), DPP_QUAD_XOR2, 0xF, 0xF, false));
  return v;
}
template <int LP>
__device__ __forceinline__ double group_sum_d(double v) {
  static_assert(LP == 4 || LP == 8, "lane group of 4 or 8");
  if constexpr (LP == 4) return quad_sum_d(v);
  else return octet_sum_d(v);
}

// Householder QR (LAPACK dlarfg convention: H = I - tau v v^T, v[0] = 1,
// H x = beta e_0) of an nrows x ncols matrix stored column-major in LDS with
// column stride ld; nref reflectors. On return the upper triangle holds R,
// the part below the diagonal v (without its unit head) and tau[j] the
// scalars. Quad qid owns the columns qid, qid + NTC/4, ...; lane q of a quad
// holds rows q, q+4, q+8, ... (RQ of them). The owner of column j+1 builds
// reflector j+1 as soon as it has applied reflector j (one barrier per
// reflector). ld should be 4 mod 32 so that the columns of different quads
// start in different banks.
template <int NTC, int RQ, bool FULL>
__device__ __forceinline__ void house_qr(float *A, int ld, int nrows, int ncols, int nref, float *tau) {
  // FULL: nrows == 4 RQ, so every row q + 4e exists. Then every load and
  // store is unconditional (masking is arithmetic: v is zero above the
  // diagonal, rows above it are written back unchanged), which lets a lane
  // issue all RQ loads of a column back to back instead of one per branch.
  constexpr int NQD = NTC / 4;
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
      while (col <= j) col += NQD;
      for (; col < ncols; col += NQD) {
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
    if (j + 1 < nref && qid == ((j + 1) & (NQD - 1))) reflector(j + 1);
    __syncthreads();
  }
}

// Matrix-core products. v_mfma_f32_16x16x4_f32 and v_mfma_f64_16x16x4_f64
// take, from lane l of the wavefront, A[l % 16][l / 16] and B[l / 16][l % 16]
// of one 16 x 16 x 4 step. Element v of lane l's accumulator then holds
// D[4 (l / 16) + v][l % 16] (fp32) or D[l / 16 + 4 v][l % 16] (fp64).
typedef __attribute__((ext_vector_type(4))) float mf32x4;
typedef __attribute__((ext_vector_type(4))) double mf64x4;

__device__ __forceinline__ mf32x4 mfma4_f32(float a, float b, mf32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ mf64x4 mfma4_f64(double a, double b, mf64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// sum_k a(i, k) b(k, j) over the 16 x 16 tiles covering M x N, in fp32 on
// matrix cores; the NW waves of the workgroup take the tiles in turn. fa / fb
// are called for i < 16 ceil(M/16), k < 16 ceil(K/16), j < 16 ceil(N/16) and
// return 0 outside the matrices. epi(i0, j0, acc) is called by the whole
// wave for each tile (lane l holds rows i0 + 4 (l/16) + v, column j0 + l%16).
// Two accumulation chains (even and odd K steps) keep consecutive
// matrix-core operations independent.
template <int NW, typename FA, typename FB, typename FE>
__device__ __forceinline__ void mfma_gemm_tiles_f32(int M, int N, int K, FA fa, FB fb, FE epi) {
  const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63, l16 = ln & 15, lk = ln >> 4;
  const int tn = (N + 15) >> 4, nt = ((M + 15) >> 4) * tn;
  for (int t = wv; t < nt; t += NW) {
    const int ti = t / tn;
    const int i0 = 16 * ti, j0 = 16 * (t - ti * tn);
    mf32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    // four K steps per iteration, their operands loaded before the first
    // product (steps past K multiply zeros; matrix-core loops are not
    // unrolled by the compiler)
    for (int k0 = 0; k0 < K; k0 += 16) {
      float av[4], bv[4];
#pragma unroll
      for (int z = 0; z < 4; z++) {
        av[z] = fa(i0 + l16, k0 + 4 * z + lk);
        bv[z] = fb(k0 + 4 * z + lk, j0 + l16);
      }
      c0 = mfma4_f32(av[0], bv[0], c0);
      c1 = mfma4_f32(av[1], bv[1], c1);
      c0 = mfma4_f32(av[2], bv[2], c0);
      c1 = mfma4_f32(av[3], bv[3], c1);
    }
    epi(i0, j0, c0 + c1);
  }
}

// the same, with out(i, j, value) called for every position of every tile
// (it checks i < M, j < N itself)
template <int NW, typename FA, typename FB, typename FO>
__device__ __forceinline__ void mfma_gemm_f32(int M, int N, int K, FA fa, FB fb, FO out) {
  const int ln = threadIdx.x & 63, l16 = ln & 15, lk = ln >> 4;
  mfma_gemm_tiles_f32<NW>(M, N, K, fa, fb, [&](int i0, int j0, mf32x4 acc) {
#pragma unroll
    for (int v = 0; v < 4; v++) out(i0 + 4 * lk + v, j0 + l16, acc[v]);
  });
}

// One-sided Jacobi over the c columns of J (column stride sj; LP lanes per
// column pair, lane o holding the contiguous rows o * 4NQ .. o * 4NQ + 4NQ - 1;
// rows past the column length are zero) without accumulating the rotations:
// on convergence the columns are mutually orthogonal (J V with V orthogonal).
// Cosines come from fp64 dot products. The squared column norms (fp64, in
// nrm) are measured at the start of every sweep and carried through each
// rotation by its exact effect on the two norms, so a pair costs one dot
// product. A pair is rotated while its cosine exceeds tol and neither column
// is negligible (squared norm <= negl: rounding noise of the matrix).
// (Taking the early sweeps' dot products in fp32 was tried: the sweeps it
// adds cost more than it saves.)

// rotation of the pair (ci, cj) by the lane group whose lane o is calling;
// returns 1 if the pair was rotated (the same on all lanes of the group)
template <int LP, int NQ>
__device__ __forceinline__ int jacobi_pair(float *J, double *nrm, int sj, int ci, int cj, int o, double tol,
                                           double negl) {
  const int rl = 4 * NQ;
  float4 *zi = (float4 *)(J + (size_t)ci * sj + o * rl);
  float4 *zj = (float4 *)(J + (size_t)cj * sj + o * rl);
  float4 xi[NQ], xj[NQ];
  const double al = nrm[ci], be = nrm[cj];
  double g[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int e = 0; e < NQ; e++) {
    xi[e] = zi[e];
    xj[e] = zj[e];
  }
#pragma unroll
  for (int e = 0; e < NQ; e++) {
    g[0] = fma((double)xi[e].x, (double)xj[e].x, g[0]);
    g[1] = fma((double)xi[e].y, (double)xj[e].y, g[1]);
    g[2] = fma((double)xi[e].z, (double)xj[e].z, g[2]);
    g[3] = fma((double)xi[e].w, (double)xj[e].w, g[3]);
  }
  const double ga = group_sum_d<LP>((g[0] + g[1]) + (g[2] + g[3]));
  if (!(al > negl && be > negl && ga * ga > tol * tol * (al * be))) return 0;
  // The rotation only has to be exact (cs^2 + sn^2 = 1 to rounding), not its
  // angle: a slightly different angle leaves a cosine the next sweep removes.
  // So the hardware reciprocal and reciprocal square root (about 1 ulp) take
  // the place of correctly rounded ones.
  const float zeta = (float)(be - al) * __builtin_amdgcn_rcpf((float)(2.0 * ga));
  const float az = fabsf(zeta);
  float t = __builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(fmaf(az, az, 1.f)));
  t = copysignf(t, zeta);
  const float cs = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f));
  const float sn = cs * t;
#pragma unroll
  for (int e = 0; e < NQ; e++) {
    const float4 u0 = xi[e], u1 = xj[e];
    zi[e] = float4{cs * u0.x - sn * u1.x, cs * u0.y - sn * u1.y, cs * u0.z - sn * u1.z, cs * u0.w - sn * u1.w};
    zj[e] = float4{sn * u0.x + cs * u1.x, sn * u0.y + cs * u1.y, sn * u0.z + cs * u1.z, sn * u0.w + cs * u1.w};
  }
  if (o == 0) {
    const double c_ = cs, s_ = sn, cg = 2.0 * c_ * s_ * ga;
    nrm[ci] = fmax(c_ * c_ * al - cg + s_ * s_ * be, 0.0);
    nrm[cj] = fmax(s_ * s_ * al + cg + c_ * c_ * be, 0.0);
  }
  return 1;
}

// squared column norms in fp64 (lane groups take the columns in turn)
template <int NTC, int LP, int NQ>
__device__ __forceinline__ void jacobi_norms(const float *J, double *nrm, int sj, int c) {
  const int tid = threadIdx.x, o = tid % LP, gid = tid / LP;
  for (int col = gid; col < c; col += NTC / LP) {
    const float4 *zc = (const float4 *)(J + (size_t)col * sj + o * 4 * NQ);
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int e = 0; e < NQ; e++) {
      const float4 x = zc[e];
      s0 = fma((double)x.x, (double)x.x, s0);
      s1 = fma((double)x.y, (double)x.y, s1);
      s0 = fma((double)x.z, (double)x.z, s0);
      s1 = fma((double)x.w, (double)x.w, s1);
    }
    const double sn2 = group_sum_d<LP>(s0 + s1);
    if (o == 0) nrm[col] = sn2;
  }
}

// workgroup sum of one int per thread (red: one LDS int, free on entry and
// on return); every thread gets the sum
template <int NTC>
__device__ __forceinline__ int block_sum_int(int v, int *red) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if (threadIdx.x == 0) *red = 0;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) atomicAdd(red, v);
  __syncthreads();
  const int s = *red;
  __syncthreads();
  return s;
}

// One cyclic sweep in the parallel round-robin order (a lane group owns one
// pair per round, one barrier per round); returns the number of rotations.
template <int NTC, int LP, int NQ>
__device__ __forceinline__ int jacobi_sweep(float *J, double *nrm, int sj, int c, double tol, double negl,
                                            int *red) {
  constexpr int NG = NTC / LP;  // lane groups; c <= 2 NG, so a group owns at most one pair per round
  const int tid = threadIdx.x, o = tid % LP, gid = tid / LP;
  const int c2 = c + (c & 1), mdl = c2 - 1;
  const bool has_pair = gid < c2 / 2;
  jacobi_norms<NTC, LP, NQ>(J, nrm, sj, c);
  __syncthreads();
  int rot = 0;
  // round-robin players of this group's pair, advanced by one each round
  // (the order of rr_pair without its two modulo operations per round)
  int pa = gid == 0 ? 0 : gid, pb = gid == 0 ? c2 - 1 : mdl - gid;
  for (int rnd = 0; rnd < c2 - 1; rnd++) {
    const int ci = pa < pb ? pa : pb, cj = pa < pb ? pb : pa;
    if (has_pair && cj < c) rot += jacobi_pair<LP, NQ>(J, nrm, sj, ci, cj, o, tol, negl);
    if (gid == 0) {
      pa++;
    } else {
      pa = (pa + 1 == mdl) ? 0 : pa + 1;
      pb = (pb + 1 == mdl) ? 0 : pb + 1;
    }
    __syncthreads();
  }
  return block_sum_int<NTC>(o == 0 ? rot : 0, red);
}

// round of the parallel round-robin order (jacobi_sweep) in which the pair
// i < j meets: player c2 - 1 meets player rnd in round rnd; otherwise the
// players of round rnd sum to 2 rnd modulo the odd c2 - 1
__device__ __forceinline__ int rr_round(int i, int j, int c2) {
  const int mdl = c2 - 1;
  if (j == mdl) return i;
  return (int)(((unsigned)(i + j) * (unsigned)((mdl + 1) / 2)) % (unsigned)mdl);
}

// The convergence test of a sweep without its sweep: the Gram matrix of the
// columns in fp64 on matrix cores (the tiles of one triangle, rows padded to
// 32 NQ with zeros), after measuring the norms afresh. Every pair i < j whose
// cosine exceeds tol (neither column negligible) sets bit j of row i of
// flags (c rows of ceil(c / 32) words) and the bit of its round-robin round
// in rmask (4 words). Returns the number of such pairs: a sweep from this
// state would rotate exactly these pairs if it met them first, and none if
// there are none.
template <int NTC, int LP, int NQ>
__device__ __forceinline__ int jacobi_flags(const float *J, double *nrm, int sj, int c, double tol, double negl,
                                            uint32_t *flags, uint32_t *rmask, int *red) {
  constexpr int NW = NTC / 64;
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63, l16 = ln & 15, lk = ln >> 4;
  const int W = (c + 31) >> 5, c2 = c + (c & 1);
  jacobi_norms<NTC, LP, NQ>(J, nrm, sj, c);
  for (int idx = tid; idx < c * W; idx += NTC) flags[idx] = 0u;
  if (tid < 4) rmask[tid] = 0u;
  __syncthreads();
  int n = 0;
  const int tk = (c + 15) >> 4;
  for (int t = wv; t < tk * (tk + 1) / 2; t += NW) {
    int tj, ti;
    tri_index(t, tj, ti);  // ti <= tj
    const int ia = 16 * ti + l16, jb = 16 * tj + l16;
    const float *ca = J + (size_t)(ia < c ? ia : 0) * sj, *cb = J + (size_t)(jb < c ? jb : 0) * sj;
    const bool va = ia < c, vb = jb < c;
    mf64x4 acc = {0.0, 0.0, 0.0, 0.0};
    for (int k0 = 0; k0 < 32 * NQ; k0 += 16) {
      double x[4], y[4];
#pragma unroll
      for (int z = 0; z < 4; z++) {
        x[z] = va ? (double)ca[k0 + 4 * z + lk] : 0.0;
        y[z] = vb ? (double)cb[k0 + 4 * z + lk] : 0.0;
      }
#pragma unroll
      for (int z = 0; z < 4; z++) acc = mfma4_f64(x[z], y[z], acc);
    }
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int i = 16 * ti + lk + 4 * v, j = jb;  // fp64 accumulator layout
      if (i < j && j < c) {
        const double g = acc[v], al = nrm[i], be = nrm[j];
        if (al > negl && be > negl && g * g > tol * tol * (al * be)) {
          atomicOr(&flags[i * W + (j >> 5)], 1u << (j & 31));
          const int rnd = rr_round(i, j, c2);
          atomicOr(&rmask[rnd >> 5], 1u << (rnd & 31));
          n++;
        }
      }
    }
  }
  return block_sum_int<NTC>(n, red);
}

// Rotates the flagged pairs: the rounds of the round-robin order that hold a
// flagged pair, in order, each lane group rotating its pair of the round if
// that pair is flagged (the rounds of a sweep, restricted to these pairs).
template <int NTC, int LP, int NQ>
__device__ __forceinline__ void jacobi_targeted(float *J, double *nrm, int sj, int c, double tol, double negl,
                                                const uint32_t *flags, const uint32_t *rmask) {
  const int tid = threadIdx.x, o = tid % LP, gid = tid / LP;
  const int W = (c + 31) >> 5, c2 = c + (c & 1), mdl = c2 - 1;
  const bool has_pair = gid < c2 / 2;
  for (int w = 0; w < 4; w++) {
    uint32_t m = rmask[w];  // the same on every thread
    while (m) {
      const int rnd = 32 * w + __builtin_ctz(m);
      m &= m - 1;
      int pa, pb;
      if (gid == 0) {
        pa = rnd;
        pb = mdl;
      } else {
        pa = (rnd + gid) % mdl;
        pb = (rnd - gid + mdl) % mdl;
      }
      const int ci = pa < pb ? pa : pb, cj = pa < pb ? pb : pa;
      if (has_pair && cj < c && ((flags[ci * W + (cj >> 5)] >> (cj & 31)) & 1u))
        jacobi_pair<LP, NQ>(J, nrm, sj, ci, cj, o, tol, negl);
      __syncthreads();
    }
  }
}

// Sweeps until one rotates nothing, or, once a sweep rotates few pairs (at
// most 4c), until the Gram test finds nothing to rotate: after such a sweep,
// the pairs the test flags are rotated directly (jacobi_targeted) and the
// test repeated, at most four times before whole sweeps resume. sweep counts
// whole sweeps and direct passes; conv is false if SWEEP_CAP was reached.
// flags: c * ceil(c/32) words, rmask: 4 words, red: one int.
template <int NTC, int LP, int NQ>
__device__ __forceinline__ void jacobi_columns(float *J, double *nrm, int sj, int c, double tol, double negl,
                                               int &sweep, bool &conv, uint32_t *flags, uint32_t *rmask,
                                               int *red) {
  while (!conv && sweep < SWEEP_CAP) {
    sweep++;
    const int nrot = jacobi_sweep<NTC, LP, NQ>(J, nrm, sj, c, tol, negl, red);
    if (nrot == 0) {
      conv = true;
      break;
    }
    if (nrot > 4 * c) continue;
    for (int pass = 0; pass < 4 && !conv && sweep < SWEEP_CAP; pass++) {
      if (jacobi_flags<NTC, LP, NQ>(J, nrm, sj, c, tol, negl, flags, rmask, red) == 0) {
        conv = true;
        break;
      }
      sweep++;
      jacobi_targeted<NTC, LP, NQ>(J, nrm, sj, c, tol, negl, flags, rmask);
    }
  }
}

}  // namespace fold
}  // namespace iskv
