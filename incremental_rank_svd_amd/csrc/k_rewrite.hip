// History coordinate rewrite: C[0:n, 0:k+] <- C[0:n, 0:k] H_top, in place.
//
// Page "iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental
// SVD", section "Block-Incremental Decoding Updates", equation for U+: every
// stored row is re-expressed in the new basis ([U 0; 0 I] G, here applied to
// C = U Sigma as C H_top, see k_core.hip). Columns k+ .. r-1 are written as
// zero, so every stored row is always r wide and clean.
//
// This is the HBM stream of a fold: each row is read once and written once.
// A workgroup owns a tile of rows, so the in-place update is race free (the
// tile is staged in LDS before any row of it is written).
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int TILE = 64;  // rows per workgroup iteration

// XK (0 keys, 1 values) is a template constant so that every access to the
// kernel arguments has a constant offset.
template <typename TC, int XK>
__device__ __forceinline__ void rewrite_body(const RewriteArgs &a, float *sm) {
  const Stream &X = a.X[XK];
  const int k = a.k[XK], kp = a.kp[XK], r = a.r[XK];
  if (a.n <= 0 || k <= 0) return;
  const int ldx = k + 1;  // padded row stride of the staged tile
  float *Hs = sm;                    // k x kp
  float *Xs = sm + (size_t)k * kp;   // TILE x ldx
  const int u = a.u0 + blockIdx.y;
  const float *Ht = X.Htop + (size_t)u * r * r;
  for (int idx = threadIdx.x; idx < k * kp; idx += NT) {
    const int i = idx / kp, j = idx - i * kp;
    Hs[idx] = Ht[(size_t)i * r + j];
  }
  TC *C = (TC *)X.C + (size_t)u * X.cstride;
  const int row_l = threadIdx.x & (TILE - 1);
  const int cg = threadIdx.x / TILE;  // 4 column groups
  for (int t0 = blockIdx.x * TILE; t0 < a.n; t0 += gridDim.x * TILE) {
    const int nrow = min(TILE, a.n - t0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nrow * k; idx += NT) {
      const int i = idx / k, j = idx - i * k;
      Xs[i * ldx + j] = ldf<TC>(C, (size_t)(t0 + i) * r + j);
    }
    __syncthreads();
    if (row_l < nrow) {
      const float *x = Xs + row_l * ldx;
      TC *crow = C + (size_t)(t0 + row_l) * r;
      for (int j0 = cg; j0 < r; j0 += 4 * 8) {
        float acc[8];
#pragma unroll
        for (int z = 0; z < 8; z++) acc[z] = 0.f;
        for (int i = 0; i < k; i++) {
          const float xv = x[i];
#pragma unroll
          for (int z = 0; z < 8; z++) {
            const int j = j0 + 4 * z;
            if (j < kp) acc[z] += xv * Hs[i * kp + j];
          }
        }
#pragma unroll
        for (int z = 0; z < 8; z++) {
          const int j = j0 + 4 * z;
          if (j < r) stf<TC>(crow, j, (j < kp) ? acc[z] : 0.f);
        }
      }
    }
  }
}

template <typename TC>
__global__ void __launch_bounds__(NT) k_rewrite_vec(const RewriteArgs a) {
  extern __shared__ float sm[];
  if (blockIdx.z == 0)
    rewrite_body<TC, 0>(a, sm);
  else
    rewrite_body<TC, 1>(a, sm);
}

// ---------------------------------------------------------------------------
// bf16 coordinates (rank a multiple of 8): matrix cores.
//
// v_mfma_f32_16x16x32_bf16 computes D (16 x 16) = A (16 x 32) . B (32 x 16):
//   A = H_top^T tile: output columns j (rows of A) x old columns (K),
//   B = C^T tile: old columns (K) x 16 stored rows; lane l holds 16
//       contiguous bytes of row l % 16, columns 8 (l / 16) .. +7, i.e. a
//       plain coalesced load of the row,
//   D: lane l holds output columns 4 (l / 16) .. +3 of row l % 16, stored as
//       one 8-byte write.
// H_top is fp32; it enters as three bf16 parts (hi + mid + lo, about 24 bits),
// so the product is accurate to fp32 rounding before the bf16 store.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int RG = 2;  // 16-row groups in flight per wavefront

template <int XK>
__device__ __forceinline__ void rewrite_mfma_body(const RewriteArgs &a, u32x4_t *fr) {
  const Stream &X = a.X[XK];
  const int k = a.k[XK], kp = a.kp[XK], r = a.r[XK];
  if (a.n <= 0 || k <= 0) return;
  const int S = (k + 31) / 32;  // K steps
  const int T = (r + 15) / 16;  // output column tiles (columns kp .. r-1 come out zero)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int u = a.u0 + blockIdx.y;
  const float *Ht = X.Htop + (size_t)u * r * r;
  // fragment (t, s, part) of lane l: H[32s + 8(l/16) + e][16t + l%16], e < 8
  for (int f = wv; f < T * S; f += NT / 64) {
    const int t = f / S, s = f - t * S;
    const int j = 16 * t + (lane & 15);
    const int kb = 32 * s + 8 * (lane >> 4);
    uint32_t w0[4], w1[4], w2[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint16_t p0[2], p1[2], p2[2];
#pragma unroll
      for (int z = 0; z < 2; z++) {
        const int kk = kb + e + z;
        const float h = (kk < k && j < kp) ? Ht[(size_t)kk * r + j] : 0.f;
        p0[z] = f2bf(h);
        const float r1 = h - bf2f(p0[z]);
        p1[z] = f2bf(r1);
        p2[z] = f2bf(r1 - bf2f(p1[z]));
      }
      w0[e / 2] = (uint32_t)p0[0] | ((uint32_t)p0[1] << 16);
      w1[e / 2] = (uint32_t)p1[0] | ((uint32_t)p1[1] << 16);
      w2[e / 2] = (uint32_t)p2[0] | ((uint32_t)p2[1] << 16);
    }
    fr[(f * 3 + 0) * 64 + lane] = u32x4_t{w0[0], w0[1], w0[2], w0[3]};
    fr[(f * 3 + 1) * 64 + lane] = u32x4_t{w1[0], w1[1], w1[2], w1[3]};
    fr[(f * 3 + 2) * 64 + lane] = u32x4_t{w2[0], w2[1], w2[2], w2[3]};
  }
  __syncthreads();
  uint16_t *C = (uint16_t *)X.C + (size_t)u * X.cstride;
  const int ngroups = (a.n + 15) / 16;
  const int gstride = gridDim.x * (NT / 64);
  for (int g0 = blockIdx.x * (NT / 64) + wv; g0 < ngroups; g0 += RG * gstride) {
    // every row of these groups is read before any of them is written
    u32x4_t cf[RG][4];
#pragma unroll
    for (int q = 0; q < RG; q++) {
      const int row = (g0 + q * gstride) * 16 + (lane & 15);
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const int kb = 32 * s + 8 * (lane >> 4);
        cf[q][s] = u32x4_t{0u, 0u, 0u, 0u};
        if (s < S && row < a.n && kb < r)
          cf[q][s] = *reinterpret_cast<const u32x4_t *>(C + (size_t)row * r + kb);
      }
    }
#pragma unroll
    for (int q = 0; q < RG; q++) {
      const int row = (g0 + q * gstride) * 16 + (lane & 15);
      for (int t = 0; t < T; t++) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++) {
          if (s < S) {
            const u32x4_t *fp = fr + (size_t)((t * S + s) * 3) * 64 + lane;
            acc = mfma_bf16(fp[0], cf[q][s], acc);
            acc = mfma_bf16(fp[64], cf[q][s], acc);
            acc = mfma_bf16(fp[128], cf[q][s], acc);
          }
        }
        const int j0 = 16 * t + 4 * (lane >> 4);
        if (row < a.n && j0 < r) {
          const uint32_t lo = (uint32_t)f2bf(acc[0]) | ((uint32_t)f2bf(acc[1]) << 16);
          const uint32_t hi = (uint32_t)f2bf(acc[2]) | ((uint32_t)f2bf(acc[3]) << 16);
          *reinterpret_cast<uint2 *>(C + (size_t)row * r + j0) = uint2{lo, hi};
        }
      }
    }
  }
}

__global__ void __launch_bounds__(NT) k_rewrite_mfma(const RewriteArgs a) {
  extern __shared__ u32x4_t fr[];
  if (blockIdx.z == 0)
    rewrite_mfma_body<0>(a, fr);
  else
    rewrite_mfma_body<1>(a, fr);
}

}  // namespace

hipError_t launch_rewrite(const RewriteArgs &a, int nunits, int coord_bf16, hipStream_t s) {
  if (a.n <= 0 || nunits <= 0) return hipSuccess;
  if (coord_bf16 && a.r[0] % 8 == 0 && a.r[1] % 8 == 0) {
    size_t lds = 0;
    for (int x = 0; x < 2; x++) {
      const size_t l = (size_t)((a.r[x] + 15) / 16) * ((a.k[x] + 31) / 32) * 3 * 64 * 16;
      if (l > lds) lds = l;
    }
    // about 512 rows per workgroup, at most 64 workgroups per unit
    int tiles = (a.n + 511) / 512;
    if (tiles > 64) tiles = 64;
    hipError_t e = hipFuncSetAttribute((const void *)k_rewrite_mfma,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rewrite_mfma, dim3(tiles, nunits, 2), dim3(NT), lds, s, a);
    return hipGetLastError();
  }
  size_t lds = 0;
  for (int x = 0; x < 2; x++) {
    const size_t l = sizeof(float) * ((size_t)a.k[x] * a.kp[x] + (size_t)TILE * (a.k[x] + 1));
    if (l > lds) lds = l;
  }
  int tiles = (a.n + TILE - 1) / TILE;
  if (tiles > 64) tiles = 64;
  dim3 grid(tiles, nunits, 2);
  if (coord_bf16) {
    hipError_t e = hipFuncSetAttribute((const void *)k_rewrite_vec<uint16_t>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rewrite_vec<uint16_t>, grid, dim3(NT), lds, s, a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void *)k_rewrite_vec<float>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rewrite_vec<float>, grid, dim3(NT), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace iskv
