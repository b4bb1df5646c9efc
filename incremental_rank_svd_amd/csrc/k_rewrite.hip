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
// so the product is accurate to fp32 rounding before the bf16 store (with two
// parts, values far below their row's norm can land more than one bf16 ulp
// from the correctly rounded product).
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// two fp32 values to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 16-row groups in flight per wavefront (each H fragment serves all of them):
// four, three for the largest ranks, whose registers would not fit two waves
// per SIMD otherwise
template <int T>
constexpr int row_groups() { return T >= 7 ? 3 : 4; }
constexpr int HP = 3;  // bf16 parts of H_top

// T = ceil(r / 16) output column tiles (columns kp .. r-1 come out zero) is a
// template constant, so that a rank's register arrays hold only its own
// tiles and K steps (at most ceil(T / 2)).
template <int T, int XK>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) k_rewrite_mfma(const RewriteArgs a) {
  extern __shared__ u32x4_t fr[];
  constexpr int SM = (T + 1) / 2;
  constexpr int RG = row_groups<T>();
  const Stream &X = a.X[XK];
  const int k = a.k[XK], kp = a.kp[XK], r = a.r[XK];
  if (a.n <= 0 || k <= 0) return;
  const int S = (k + 31) / 32;  // K steps, at most SM
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
    fr[(f * HP + 0) * 64 + lane] = u32x4_t{w0[0], w0[1], w0[2], w0[3]};
    fr[(f * HP + 1) * 64 + lane] = u32x4_t{w1[0], w1[1], w1[2], w1[3]};
    fr[(f * HP + 2) * 64 + lane] = u32x4_t{w2[0], w2[1], w2[2], w2[3]};
  }
  __syncthreads();
  uint16_t *C = (uint16_t *)X.C + (size_t)u * X.cstride;
  const int ngroups = (a.n + 15) / 16;
  const int gstride = gridDim.x * (NT / 64);
  // The unit's rows are read and written through a buffer resource whose
  // range is the n stored rows: an access past it reads zeros and writes
  // nothing, so rows past n and 16-byte chunks past column r (their offset is
  // pushed above 2^31, out of the range) need no branch and no select.
  // The RG groups of the next iteration are loaded while the current ones are
  // computed (their rows are disjoint from the rows being written).
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(C, (short)0, a.n * r * 2, 0x00020000);
  // (offsets are unsigned 32-bit; the launcher keeps every row offset below 2^31)
  constexpr uint32_t OUT = 0x80000000u;
  const int kq = 8 * (lane >> 4), jq = 4 * (lane >> 4);
  auto coff = [&](int s) { return 32 * s + kq < r ? 2u * (32 * s + kq) : OUT; };
  // Output staging: one 16-row group per wave in LDS after the fragments,
  // rows RS bytes apart (room for T whole tiles plus 16 bytes against bank
  // conflicts). A lane writes its 8-byte pieces of a row there, then the
  // group (16 rows of 2r bytes, contiguous in memory) is read back and
  // stored as 16 contiguous bytes per lane: whole lines per instruction.
  constexpr int RS = 32 * T + 16, NI = (T + 1) / 2;  // 16 * 32T bytes <= NI KiB
  char *stg = reinterpret_cast<char *>(fr + (size_t)T * S * HP * 64) + wv * 16 * RS;
  char *stw = stg + (lane & 15) * RS + 2 * jq;
  uint32_t sl[NI], so[NI];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int off = 1024 * i + 16 * lane, row = off / (2 * r), col = off - row * 2 * r;
    const bool in = off < 32 * r;
    sl[i] = in ? row * RS + col : 0;
    so[i] = in ? (uint32_t)off : OUT;
  }
  auto load_groups = [&](int g0, u32x4_t (&cf)[RG][SM]) {
#pragma unroll
    for (int q = 0; q < RG; q++) {
      const uint32_t ro = (uint32_t)((g0 + q * gstride) * 16 + (lane & 15)) * (uint32_t)(2 * r);
#pragma unroll
      for (int s = 0; s < SM; s++)
        cf[q][s] = s < S ? __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(ro + coff(s)), 0, 0)
                         : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  u32x4_t cf[RG][SM], cn[RG][SM];
  const int gfirst = blockIdx.x * (NT / 64) + wv;
  if (gfirst < ngroups) load_groups(gfirst, cn);
  for (int g0 = gfirst; g0 < ngroups; g0 += RG * gstride) {
#pragma unroll
    for (int q = 0; q < RG; q++)
#pragma unroll
      for (int s = 0; s < SM; s++) cf[q][s] = cn[q][s];
    if (g0 + RG * gstride < ngroups) load_groups(g0 + RG * gstride, cn);
    // each H fragment is read from LDS once for all RG groups; the output
    // tiles stay in registers until all T are done, then each group goes to
    // memory through the wave's LDS staging rows as whole contiguous rows
    u32x2_t ob[RG][T];
#pragma unroll
    for (int t = 0; t < T; t++) {
      {
        f32x4_t acc[RG];
#pragma unroll
        for (int q = 0; q < RG; q++) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SM; s++) {
          if (s < S) {
            const u32x4_t *fp = fr + (size_t)((t * S + s) * HP) * 64 + lane;
#pragma unroll
            for (int part = 0; part < HP; part++) {
              const u32x4_t f = fp[64 * part];
#pragma unroll
              for (int q = 0; q < RG; q++) acc[q] = mfma_bf16(f, cf[q][s], acc[q]);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < RG; q++) ob[q][t] = u32x2_t{pack_bf16(acc[q][0], acc[q][1]), pack_bf16(acc[q][2], acc[q][3])};
        // keep the scheduler from overlapping tiles (each tile's accumulators
        // would stay live, and the registers of large ranks run out)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int q = 0; q < RG; q++) {
#pragma unroll
      for (int t = 0; t < T; t++) *reinterpret_cast<u32x2_t *>(stw + 32 * t) = ob[q][t];
      // other lanes of this wave read what it wrote (a wave's LDS accesses
      // complete in order; the fences keep the compiler from moving them)
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const uint32_t go = (uint32_t)(g0 + q * gstride) * (uint32_t)(32 * r);
#pragma unroll
      for (int i = 0; i < NI; i++)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t *>(stg + sl[i]), rs,
                                               (int)(go + so[i]), 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
  }
}

template <int T>
hipError_t launch_rewrite_t(const RewriteArgs &a, int x, dim3 grid, size_t lds, hipStream_t s) {
  const void *f = x == 0 ? (const void *)k_rewrite_mfma<T, 0> : (const void *)k_rewrite_mfma<T, 1>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (x == 0)
    hipLaunchKernelGGL((k_rewrite_mfma<T, 0>), grid, dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL((k_rewrite_mfma<T, 1>), grid, dim3(NT), lds, s, a);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// int8 storage (codes of U = C Sigma^-1, one fp32 scale per row): every stored
// row becomes u M in place, M = Sigma_old H_top Sigma_new^-1 (k x k+, fp32, in
// the Htop scratch). A row's codes enter the bf16 matrix-core product exactly
// (|q| <= 127) and its old scale factors out, so the product a = q M gives the
// new codes rint(127 a / max|a|) and the new scale s_old max|a| / 127. Same
// scheme as k_rewrite_mfma: three bf16 parts of M in LDS fragments, RG 16-row
// groups per wave with the next ones loading; per K step lane l loads the 8
// codes of columns 8 (l / 16) .. +7 of row l % 16 and widens them to bf16 in
// registers. A row's outputs sit in the four lanes l % 16 of each tile, so its
// maximum takes two shuffles; the codes (4 bytes per lane and tile) go through
// a per-wave LDS copy of the group (16 r contiguous bytes, unpadded, in memory
// order) and leave as whole 16-byte pieces.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2v_t;

template <int T, int XK>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) k_rewrite_i8(const RewriteArgs a) {
  extern __shared__ u32x4_t fr[];
  constexpr int SM = (T + 1) / 2;
  constexpr int RG = row_groups<T>();
  const Stream &X = a.X[XK];
  const int k = a.k[XK], kp = a.kp[XK], r = a.r[XK];
  if (a.n <= 0 || k <= 0) return;
  const int S = (k + 31) / 32;  // K steps, at most SM
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int u = a.u0 + blockIdx.y;
  const float *Ht = X.Htop + (size_t)u * r * r;
  // The K order of the products is permuted so that lane l loads 16
  // contiguous codes, columns 64 p + 16 (l / 16) .. +15 of its row, for each
  // whole pair p of K steps (whole 16-row groups per load instruction): step
  // s takes the half s % 2 of pair s / 2. A last unpaired step (S odd) loads
  // 8 codes, columns 32 s + 8 (l / 16) .. +7. The fragments of M follow the
  // same order: fragment (t, s, part) of lane l holds M[kb + e][16t + l%16],
  // e < 8, kb = 64 (s/2) + 16 (l/16) + 8 (s%2) in a pair, else 32 s + 8 (l/16).
  for (int f = wv; f < T * S; f += NT / 64) {
    const int t = f / S, s = f - t * S;
    const int j = 16 * t + (lane & 15);
    const int kb = (s | 1) < S ? 64 * (s >> 1) + 16 * (lane >> 4) + 8 * (s & 1) : 32 * s + 8 * (lane >> 4);
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
    fr[(f * HP + 0) * 64 + lane] = u32x4_t{w0[0], w0[1], w0[2], w0[3]};
    fr[(f * HP + 1) * 64 + lane] = u32x4_t{w1[0], w1[1], w1[2], w1[3]};
    fr[(f * HP + 2) * 64 + lane] = u32x4_t{w2[0], w2[1], w2[2], w2[3]};
  }
  __syncthreads();
  int8_t *C = (int8_t *)X.C + (size_t)u * X.cstride;
  float *cs = X.cs + (size_t)u * cs_stride(a.ncap);
  const int ngroups = (a.n + 15) / 16;
  const int gstride = gridDim.x * (NT / 64);
  // codes and scales through buffer resources whose ranges are the n stored
  // rows: rows past n read zeros and are not written, and so are code pieces
  // past column r (offset pushed above 2^31)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, a.n * r, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(cs, (short)0, a.n * 4, 0x00020000);
  constexpr uint32_t OUT = 0x80000000u;
  const int jq = 4 * (lane >> 4);
  constexpr int SP = (SM + 1) / 2;  // K-step pairs (the last one may be a single step)
  // column of lane l's piece of pair p: 16 codes in a whole pair, 8 in a last single step
  // (a 16-code piece that starts below column r may end past it when r % 16 == 8:
  // those codes belong to the next row and meet rows of M past k, which are zero)
  auto pcol = [&](int p) { return 2 * p + 1 < S ? 64 * p + 16 * (lane >> 4) : 64 * p + 8 * (lane >> 4); };
  auto coff = [&](int p) { return pcol(p) < r ? (uint32_t)pcol(p) : OUT; };
  const bool al16 = (r & 15) == 0;  // 16-byte pieces are 16-byte aligned
  constexpr int GB = 16 * 16 * T;             // bytes of a group's staging (16 rows of at most 16 T)
  constexpr int NI = (GB + 1023) / 1024;      // 16-byte pieces per lane
  char *stg = reinterpret_cast<char *>(fr + (size_t)T * S * HP * 64) + wv * GB;
  char *stw = stg + (lane & 15) * r + jq;
  uint32_t sl[NI], so[NI];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int off = 1024 * i + 16 * lane;
    sl[i] = off < 16 * r ? (uint32_t)off : 0u;
    so[i] = off < 16 * r ? (uint32_t)off : OUT;
  }
  auto load_groups = [&](int g0, u32x4_t (&cf)[RG][SP], float (&sc)[RG]) {
#pragma unroll
    for (int q = 0; q < RG; q++) {
      const uint32_t row = (uint32_t)((g0 + q * gstride) * 16 + (lane & 15));
      const uint32_t ro = row * (uint32_t)r;
#pragma unroll
      for (int p = 0; p < SP; p++) {
        if (2 * p + 1 == S) {  // last single step: 8 codes
          const u32x2v_t lo = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(ro + coff(p)), 0, 0);
          cf[q][p] = u32x4_t{lo[0], lo[1], 0u, 0u};
        } else if (2 * p < S) {
          const int o = (int)(ro + coff(p));
          if (al16) {
            cf[q][p] = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
          } else {
            const u32x2v_t lo = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
            const u32x2v_t hi = __builtin_amdgcn_raw_buffer_load_b64(rs, o + 8, 0, 0);
            cf[q][p] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          }
        } else {
          cf[q][p] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
      sc[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsc, (int)(row * 4u), 0, 0));
    }
  };
  u32x4_t cf[RG][SP], cn[RG][SP];
  float sc[RG], scn[RG];
  const int gfirst = blockIdx.x * (NT / 64) + wv;
  if (gfirst < ngroups) load_groups(gfirst, cn, scn);
  for (int g0 = gfirst; g0 < ngroups; g0 += RG * gstride) {
    u32x4_t bq[RG][SM];
#pragma unroll
    for (int q = 0; q < RG; q++) {
      sc[q] = scn[q];
#pragma unroll
      for (int p = 0; p < SP; p++) cf[q][p] = cn[q][p];
#pragma unroll
      for (int s = 0; s < SM; s++) {
        uint32_t w[4];
        i8x8_bf16(cf[q][s >> 1][2 * (s & 1)], cf[q][s >> 1][2 * (s & 1) + 1], w);
        bq[q][s] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
    if (g0 + RG * gstride < ngroups) load_groups(g0 + RG * gstride, cn, scn);
    f32x4_t ob[RG][T];
#pragma unroll
    for (int t = 0; t < T; t++) {
#pragma unroll
      for (int q = 0; q < RG; q++) ob[q][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < SM; s++) {
        if (s < S) {
          const u32x4_t *fp = fr + (size_t)((t * S + s) * HP) * 64 + lane;
#pragma unroll
          for (int part = 0; part < HP; part++) {
            const u32x4_t f = fp[64 * part];
#pragma unroll
            for (int q = 0; q < RG; q++) ob[q][t] = mfma_bf16(f, bq[q][s], ob[q][t]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < RG; q++) {
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < T; t++)
#pragma unroll
        for (int i = 0; i < 4; i++) m = fmaxf(m, fabsf(ob[q][t][i]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      const float inv = i8_inv_step(m);
#pragma unroll
      for (int t = 0; t < T; t++) {
        if (16 * t + jq < r)
          *reinterpret_cast<uint32_t *>(stw + 16 * t) =
              i8_pack4(ob[q][t][0], ob[q][t][1], ob[q][t][2], ob[q][t][3], inv);
      }
      // other lanes of this wave read what it wrote (a wave's LDS accesses
      // complete in order; the fences keep the compiler from moving them)
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const uint32_t grow = (uint32_t)(g0 + q * gstride) * 16u;
#pragma unroll
      for (int i = 0; i < NI; i++)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t *>(stg + sl[i]), rs,
                                               (int)(grow * (uint32_t)r + so[i]), 0, 0);
      if (lane < 16)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc[q] * (m / 127.f)), rsc,
                                              (int)((grow + lane) * 4u), 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
  }
}

template <int T>
hipError_t launch_rewrite_i8_t(const RewriteArgs &a, int x, dim3 grid, size_t lds, hipStream_t s) {
  const void *f = x == 0 ? (const void *)k_rewrite_i8<T, 0> : (const void *)k_rewrite_i8<T, 1>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (x == 0)
    hipLaunchKernelGGL((k_rewrite_i8<T, 0>), grid, dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL((k_rewrite_i8<T, 1>), grid, dim3(NT), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One-shot prefill coordinates on matrix cores: C[i] = X[i] B^T for all prompt
// rows of a unit (bf16 rows and coordinates), and sigma = the column norms of
// what is stored. Page "iS-KV: Online Low-Rank KV Cache Compression via
// Block-Incremental SVD", section "Prefill Compression" (the history's
// coordinates in the truncated basis). The rewrite's scheme with the 128
// input dimensions as K (four K steps) and B^T in place of H_top: B (fp32)
// enters as three bf16 parts, each wave keeps RG 16-row groups in flight with
// the next ones loading, and outputs leave through LDS as whole rows. One
// workgroup per unit stream, so the column sums of squares reduce in a fixed
// order (lanes, then the four waves).
// ---------------------------------------------------------------------------
template <int T, int XK>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) k_coords_mfma(const OneshotArgs a) {
  extern __shared__ u32x4_t fr[];
  constexpr int S = D / 32, RG = row_groups<T>();
  const Stream &X = a.X[XK];
  const int r = X.r;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int lrel = ul / (a.batch * a.kvh), rem = ul - lrel * (a.batch * a.kvh);
  const int bi = rem / a.kvh, hh = rem - bi * a.kvh;
  const uint16_t *src = (const uint16_t *)a.src[XK] +
                        (((size_t)bi * a.nl_in + a.lrel0 + lrel) * a.kvh + hh) * (size_t)a.nrows * D;
  const int kplus = min(min(r, a.nrows), D);
  const float *Bt = X.Bt + (size_t)u * r * D;
  // fragment (t, s, part) of lane l: B^T[32s + 8(l/16) + e][16t + l%16], e < 8
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
        const float h = (j < kplus) ? Bt[(size_t)j * D + kb + e + z] : 0.f;
        p0[z] = f2bf(h);
        const float r1 = h - bf2f(p0[z]);
        p1[z] = f2bf(r1);
        p2[z] = f2bf(r1 - bf2f(p1[z]));
      }
      w0[e / 2] = (uint32_t)p0[0] | ((uint32_t)p0[1] << 16);
      w1[e / 2] = (uint32_t)p1[0] | ((uint32_t)p1[1] << 16);
      w2[e / 2] = (uint32_t)p2[0] | ((uint32_t)p2[1] << 16);
    }
    fr[(f * HP + 0) * 64 + lane] = u32x4_t{w0[0], w0[1], w0[2], w0[3]};
    fr[(f * HP + 1) * 64 + lane] = u32x4_t{w1[0], w1[1], w1[2], w1[3]};
    fr[(f * HP + 2) * 64 + lane] = u32x4_t{w2[0], w2[1], w2[2], w2[3]};
  }
  constexpr int RS = 32 * T + 16, NI = (T + 1) / 2;
  char *stg = reinterpret_cast<char *>(fr + (size_t)T * S * HP * 64) + wv * 16 * RS;
  float *sqw = reinterpret_cast<float *>(reinterpret_cast<char *>(fr + (size_t)T * S * HP * 64) + (NT / 64) * 16 * RS);
  __syncthreads();
  // prompt rows (16 bytes per lane) and coordinate rows through buffer
  // resources whose ranges are the unit's rows: rows past nrows read zeros
  // and are not written
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, a.nrows * D * 2, 0x00020000);
  uint16_t *C = (uint16_t *)X.C + (size_t)u * X.cstride;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, a.nrows * r * 2, 0x00020000);
  constexpr uint32_t OUT = 0x80000000u;
  const int jq = 4 * (lane >> 4);
  char *stw = stg + (lane & 15) * RS + 2 * jq;
  uint32_t sl[NI], so[NI];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int off = 1024 * i + 16 * lane, row = off / (2 * r), col = off - row * 2 * r;
    const bool in = off < 32 * r;
    sl[i] = in ? row * RS + col : 0;
    so[i] = in ? (uint32_t)off : OUT;
  }
  const int ngroups = (a.nrows + 15) / 16;
  constexpr int gstride = NT / 64;
  auto load_groups = [&](int g0, u32x4_t (&cf)[RG][S]) {
#pragma unroll
    for (int q = 0; q < RG; q++) {
      const uint32_t ro = (uint32_t)((g0 + q * gstride) * 16 + (lane & 15)) * (uint32_t)(2 * D) + 16u * (lane >> 4);
#pragma unroll
      for (int s = 0; s < S; s++) cf[q][s] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(ro + 64u * s), 0, 0);
    }
  };
  float sq[T][4];
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) sq[t][v] = 0.f;
  u32x4_t cf[RG][S], cn[RG][S];
  if (wv < ngroups) load_groups(wv, cn);
  for (int g0 = wv; g0 < ngroups; g0 += RG * gstride) {
#pragma unroll
    for (int q = 0; q < RG; q++)
#pragma unroll
      for (int s = 0; s < S; s++) cf[q][s] = cn[q][s];
    if (g0 + RG * gstride < ngroups) load_groups(g0 + RG * gstride, cn);
    u32x2_t ob[RG][T];
#pragma unroll
    for (int t = 0; t < T; t++) {
      f32x4_t acc[RG];
#pragma unroll
      for (int q = 0; q < RG; q++) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; s++) {
        const u32x4_t *fp = fr + (size_t)((t * S + s) * HP) * 64 + lane;
#pragma unroll
        for (int part = 0; part < HP; part++) {
          const u32x4_t f = fp[64 * part];
#pragma unroll
          for (int q = 0; q < RG; q++) acc[q] = mfma_bf16(f, cf[q][s], acc[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < RG; q++) {
        ob[q][t] = u32x2_t{pack_bf16(acc[q][0], acc[q][1]), pack_bf16(acc[q][2], acc[q][3])};
        // squares of the stored (rounded) values; rows past nrows are zero
        const float v0 = __uint_as_float(ob[q][t][0] << 16), v1 = __uint_as_float(ob[q][t][0] & 0xffff0000u);
        const float v2 = __uint_as_float(ob[q][t][1] << 16), v3 = __uint_as_float(ob[q][t][1] & 0xffff0000u);
        sq[t][0] += v0 * v0;
        sq[t][1] += v1 * v1;
        sq[t][2] += v2 * v2;
        sq[t][3] += v3 * v3;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < RG; q++) {
#pragma unroll
      for (int t = 0; t < T; t++) *reinterpret_cast<u32x2_t *>(stw + 32 * t) = ob[q][t];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const uint32_t go = (uint32_t)(g0 + q * gstride) * (uint32_t)(32 * r);
#pragma unroll
      for (int i = 0; i < NI; i++)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t *>(stg + sl[i]), rc,
                                               (int)(go + so[i]), 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
  }
  // column sums of squares: over the 16 rows of each lane group (fixed
  // butterfly), then over the four waves in order
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) {
      float x = sq[t][v];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if ((lane & 15) == 0) sqw[wv * (16 * T) + 16 * t + jq + v] = x;
    }
  __syncthreads();
  if ((int)threadIdx.x < r) {
    const int j = threadIdx.x;
    float s2 = 0.f;
    for (int w = 0; w < NT / 64; w++) s2 += sqw[w * (16 * T) + j];
    X.sig[(size_t)u * r + j] = (j < kplus) ? sqrtf(s2) : 0.f;
  }
}

// int8 storage of the one-shot history: sigma_j = norm of column j of X B^T
// (first pass over the rows, fixed-order reduction as above), then each row
// of U = X B^T Sigma^-1 is stored as int8 codes with its own scale (second
// pass, the same products again). Fragments, loads and the LDS staging of the
// outputs as in k_coords_mfma and k_rewrite_i8.
template <int T, int XK>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) k_coords_i8(const OneshotArgs a) {
  extern __shared__ u32x4_t fr[];
  constexpr int S = D / 32, RG = row_groups<T>();
  const Stream &X = a.X[XK];
  const int r = X.r;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int lrel = ul / (a.batch * a.kvh), rem = ul - lrel * (a.batch * a.kvh);
  const int bi = rem / a.kvh, hh = rem - bi * a.kvh;
  const uint16_t *src = (const uint16_t *)a.src[XK] +
                        (((size_t)bi * a.nl_in + a.lrel0 + lrel) * a.kvh + hh) * (size_t)a.nrows * D;
  const int kplus = min(min(r, a.nrows), D);
  const float *Bt = X.Bt + (size_t)u * r * D;
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
        const float h = (j < kplus) ? Bt[(size_t)j * D + kb + e + z] : 0.f;
        p0[z] = f2bf(h);
        const float r1 = h - bf2f(p0[z]);
        p1[z] = f2bf(r1);
        p2[z] = f2bf(r1 - bf2f(p1[z]));
      }
      w0[e / 2] = (uint32_t)p0[0] | ((uint32_t)p0[1] << 16);
      w1[e / 2] = (uint32_t)p1[0] | ((uint32_t)p1[1] << 16);
      w2[e / 2] = (uint32_t)p2[0] | ((uint32_t)p2[1] << 16);
    }
    fr[(f * HP + 0) * 64 + lane] = u32x4_t{w0[0], w0[1], w0[2], w0[3]};
    fr[(f * HP + 1) * 64 + lane] = u32x4_t{w1[0], w1[1], w1[2], w1[3]};
    fr[(f * HP + 2) * 64 + lane] = u32x4_t{w2[0], w2[1], w2[2], w2[3]};
  }
  constexpr int GB = 16 * 16 * T, NI = (GB + 1023) / 1024;
  char *stg = reinterpret_cast<char *>(fr + (size_t)T * S * HP * 64) + wv * GB;
  float *sqw = reinterpret_cast<float *>(reinterpret_cast<char *>(fr + (size_t)T * S * HP * 64) + (NT / 64) * GB);
  float *isg = sqw + (NT / 64) * 16 * T;  // 1 / sigma_j (0 where sigma_j = 0), 16 T floats
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, a.nrows * D * 2, 0x00020000);
  int8_t *C = (int8_t *)X.C + (size_t)u * X.cstride;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, a.nrows * r, 0x00020000);
  constexpr uint32_t OUT = 0x80000000u;
  const int jq = 4 * (lane >> 4);
  char *stw = stg + (lane & 15) * r + jq;
  uint32_t sl[NI], so[NI];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int off = 1024 * i + 16 * lane;
    sl[i] = off < 16 * r ? (uint32_t)off : 0u;
    so[i] = off < 16 * r ? (uint32_t)off : OUT;
  }
  const int ngroups = (a.nrows + 15) / 16;
  constexpr int gstride = NT / 64;
  auto load_groups = [&](int g0, u32x4_t (&cf)[RG][S]) {
#pragma unroll
    for (int q = 0; q < RG; q++) {
      const uint32_t ro = (uint32_t)((g0 + q * gstride) * 16 + (lane & 15)) * (uint32_t)(2 * D) + 16u * (lane >> 4);
#pragma unroll
      for (int s = 0; s < S; s++) cf[q][s] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(ro + 64u * s), 0, 0);
    }
  };
  auto products = [&](const u32x4_t (&cf)[RG][S], f32x4_t (&ob)[RG][T]) {
#pragma unroll
    for (int t = 0; t < T; t++) {
#pragma unroll
      for (int q = 0; q < RG; q++) ob[q][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; s++) {
        const u32x4_t *fp = fr + (size_t)((t * S + s) * HP) * 64 + lane;
#pragma unroll
        for (int part = 0; part < HP; part++) {
          const u32x4_t f = fp[64 * part];
#pragma unroll
          for (int q = 0; q < RG; q++) ob[q][t] = mfma_bf16(f, cf[q][s], ob[q][t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  u32x4_t cf[RG][S], cn[RG][S];
  // pass 1: column sums of squares of X B^T
  {
    float sq[T][4];
#pragma unroll
    for (int t = 0; t < T; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) sq[t][v] = 0.f;
    if (wv < ngroups) load_groups(wv, cn);
    for (int g0 = wv; g0 < ngroups; g0 += RG * gstride) {
#pragma unroll
      for (int q = 0; q < RG; q++)
#pragma unroll
        for (int s = 0; s < S; s++) cf[q][s] = cn[q][s];
      if (g0 + RG * gstride < ngroups) load_groups(g0 + RG * gstride, cn);
      f32x4_t ob[RG][T];
      products(cf, ob);
#pragma unroll
      for (int q = 0; q < RG; q++)
#pragma unroll
        for (int t = 0; t < T; t++)
#pragma unroll
          for (int v = 0; v < 4; v++) sq[t][v] += ob[q][t][v] * ob[q][t][v];
    }
#pragma unroll
    for (int t = 0; t < T; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        float x = sq[t][v];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if ((lane & 15) == 0) sqw[wv * (16 * T) + 16 * t + jq + v] = x;
      }
  }
  __syncthreads();
  if ((int)threadIdx.x < 16 * T) {
    const int j = threadIdx.x;
    float s2 = 0.f;
    for (int w = 0; w < NT / 64; w++) s2 += sqw[w * (16 * T) + j];
    const float sg = (j < kplus) ? sqrtf(s2) : 0.f;
    if (j < r) X.sig[(size_t)u * r + j] = sg;
    isg[j] = sg > 0.f ? 1.f / sg : 0.f;
  }
  __syncthreads();
  // pass 2: rows of U in int8 with per-row scales
  float *scl = X.cs + (size_t)u * cs_stride(a.ncap);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(scl, (short)0, a.nrows * 4, 0x00020000);
  float iv[T][4];
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) iv[t][v] = isg[16 * t + jq + v];
  if (wv < ngroups) load_groups(wv, cn);
  for (int g0 = wv; g0 < ngroups; g0 += RG * gstride) {
#pragma unroll
    for (int q = 0; q < RG; q++)
#pragma unroll
      for (int s = 0; s < S; s++) cf[q][s] = cn[q][s];
    if (g0 + RG * gstride < ngroups) load_groups(g0 + RG * gstride, cn);
    f32x4_t ob[RG][T];
    products(cf, ob);
#pragma unroll
    for (int q = 0; q < RG; q++) {
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < T; t++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          ob[q][t][v] *= iv[t][v];
          m = fmaxf(m, fabsf(ob[q][t][v]));
        }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      const float inv = i8_inv_step(m);
#pragma unroll
      for (int t = 0; t < T; t++) {
        if (16 * t + jq < r)
          *reinterpret_cast<uint32_t *>(stw + 16 * t) =
              i8_pack4(ob[q][t][0], ob[q][t][1], ob[q][t][2], ob[q][t][3], inv);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const uint32_t grow = (uint32_t)(g0 + q * gstride) * 16u;
#pragma unroll
      for (int i = 0; i < NI; i++)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t *>(stg + sl[i]), rc,
                                               (int)(grow * (uint32_t)r + so[i]), 0, 0);
      if (lane < 16)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m / 127.f), rsc, (int)((grow + lane) * 4u), 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
  }
}

template <int T>
hipError_t launch_coords_i8_t(const OneshotArgs &a, int x, int nunits, hipStream_t s) {
  const size_t lds = (size_t)T * (D / 32) * HP * 64 * 16 + (size_t)(NT / 64) * 16 * 16 * T +
                     sizeof(float) * ((NT / 64) * 16 * T + 16 * T);
  const void *f = x == 0 ? (const void *)k_coords_i8<T, 0> : (const void *)k_coords_i8<T, 1>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (x == 0)
    hipLaunchKernelGGL((k_coords_i8<T, 0>), dim3(nunits), dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL((k_coords_i8<T, 1>), dim3(nunits), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <int T>
hipError_t launch_coords_t(const OneshotArgs &a, int x, int nunits, hipStream_t s) {
  const size_t lds = (size_t)T * (D / 32) * HP * 64 * 16 + (size_t)(NT / 64) * 16 * (32 * T + 16) +
                     sizeof(float) * (NT / 64) * 16 * T;
  const void *f = x == 0 ? (const void *)k_coords_mfma<T, 0> : (const void *)k_coords_mfma<T, 1>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (x == 0)
    hipLaunchKernelGGL((k_coords_mfma<T, 0>), dim3(nunits), dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL((k_coords_mfma<T, 1>), dim3(nunits), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rewrite(const RewriteArgs &a, int nunits, int coord_bf16, hipStream_t s) {
  if (a.n <= 0 || nunits <= 0) return hipSuccess;
  // matrix-core path: bf16 rows 16-byte aligned, and every row offset the
  // kernel forms (up to n plus the rows of one prefetch, in bytes) below 2^31
  const int rmax = a.r[0] > a.r[1] ? a.r[0] : a.r[1];
  if (coord_bf16 && a.r[0] % 8 == 0 && a.r[1] % 8 == 0 &&
      ((size_t)a.n + 65536) * rmax * 2 < ((size_t)1 << 31)) {
    // about 2048 rows per workgroup (the H fragments are built once per
    // workgroup), at most 64 workgroups per unit; one launch per kind
    int tiles = (a.n + 2047) / 2048;
    if (tiles > 64) tiles = 64;
    for (int x = 0; x < 2; x++) {
      if (a.k[x] <= 0) continue;
      const int T = (a.r[x] + 15) / 16;
      const size_t lds = (size_t)T * ((a.k[x] + 31) / 32) * HP * 64 * 16 + (size_t)(NT / 64) * 16 * (32 * T + 16);
      const dim3 grid(tiles, nunits, 1);
      hipError_t e;
      switch ((a.r[x] + 15) / 16) {
        case 1: e = launch_rewrite_t<1>(a, x, grid, lds, s); break;
        case 2: e = launch_rewrite_t<2>(a, x, grid, lds, s); break;
        case 3: e = launch_rewrite_t<3>(a, x, grid, lds, s); break;
        case 4: e = launch_rewrite_t<4>(a, x, grid, lds, s); break;
        case 5: e = launch_rewrite_t<5>(a, x, grid, lds, s); break;
        case 6: e = launch_rewrite_t<6>(a, x, grid, lds, s); break;
        case 7: e = launch_rewrite_t<7>(a, x, grid, lds, s); break;
        default: e = launch_rewrite_t<8>(a, x, grid, lds, s); break;
      }
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
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

hipError_t launch_rewrite_i8(const RewriteArgs &a, int nunits, hipStream_t s) {
  if (a.n <= 0 || nunits <= 0) return hipSuccess;
  // the configuration check keeps (ncap + 65536) r below 2^31 (every offset a
  // wave forms, a prefetch past n included)
  int tiles = (a.n + 2047) / 2048;
  if (tiles > 64) tiles = 64;
  for (int x = 0; x < 2; x++) {
    if (a.k[x] <= 0) continue;
    const int T = (a.r[x] + 15) / 16;
    const size_t lds = (size_t)T * ((a.k[x] + 31) / 32) * HP * 64 * 16 + (size_t)(NT / 64) * 16 * 16 * T;
    const dim3 grid(tiles, nunits, 1);
    hipError_t e;
    switch (T) {
      case 1: e = launch_rewrite_i8_t<1>(a, x, grid, lds, s); break;
      case 2: e = launch_rewrite_i8_t<2>(a, x, grid, lds, s); break;
      case 3: e = launch_rewrite_i8_t<3>(a, x, grid, lds, s); break;
      case 4: e = launch_rewrite_i8_t<4>(a, x, grid, lds, s); break;
      case 5: e = launch_rewrite_i8_t<5>(a, x, grid, lds, s); break;
      case 6: e = launch_rewrite_i8_t<6>(a, x, grid, lds, s); break;
      case 7: e = launch_rewrite_i8_t<7>(a, x, grid, lds, s); break;
      default: e = launch_rewrite_i8_t<8>(a, x, grid, lds, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace iskv

namespace iskv {

bool oneshot_coords_mfma_ok(const OneshotArgs &a, int kv_bf16, int coord_bf16) {
  return kv_bf16 && coord_bf16 && a.X[0].r % 8 == 0 && a.X[1].r % 8 == 0 &&
         ((size_t)a.nrows + 65536) * D * 2 < ((size_t)1 << 31);
}

hipError_t launch_oneshot_coords_i8(const OneshotArgs &a, int nunits, hipStream_t s) {
  for (int x = 0; x < 2; x++) {
    hipError_t e;
    switch ((a.X[x].r + 15) / 16) {
      case 1: e = launch_coords_i8_t<1>(a, x, nunits, s); break;
      case 2: e = launch_coords_i8_t<2>(a, x, nunits, s); break;
      case 3: e = launch_coords_i8_t<3>(a, x, nunits, s); break;
      case 4: e = launch_coords_i8_t<4>(a, x, nunits, s); break;
      case 5: e = launch_coords_i8_t<5>(a, x, nunits, s); break;
      case 6: e = launch_coords_i8_t<6>(a, x, nunits, s); break;
      case 7: e = launch_coords_i8_t<7>(a, x, nunits, s); break;
      default: e = launch_coords_i8_t<8>(a, x, nunits, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_oneshot_coords_mfma(const OneshotArgs &a, int nunits, hipStream_t s) {
  for (int x = 0; x < 2; x++) {
    hipError_t e;
    switch ((a.X[x].r + 15) / 16) {
      case 1: e = launch_coords_t<1>(a, x, nunits, s); break;
      case 2: e = launch_coords_t<2>(a, x, nunits, s); break;
      case 3: e = launch_coords_t<3>(a, x, nunits, s); break;
      case 4: e = launch_coords_t<4>(a, x, nunits, s); break;
      case 5: e = launch_coords_t<5>(a, x, nunits, s); break;
      case 6: e = launch_coords_t<6>(a, x, nunits, s); break;
      case 7: e = launch_coords_t<7>(a, x, nunits, s); break;
      default: e = launch_coords_t<8>(a, x, nunits, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace iskv
