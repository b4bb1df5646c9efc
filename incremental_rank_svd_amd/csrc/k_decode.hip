// Single-token decode attention over the compressed cache.
//
// For a history row i, K~_i = C_K[i] B_K^T (section "Reconstruction and
// Storage" of the iS-KV page), so its score is
//     s_i = scale * K~_i . q = C_K[i] . q'   with   q' = scale * B_K^T q,
// and the weighted history values are (sum_i p_i C_V[i]) B_V^T. The window
// rows are used as stored. Softmax runs over history and window together,
// split over chunks of history rows and merged by log-sum-exp.
//
// One launch, grid (history chunks + 1, units):
//   - a history block computes q' for its unit, then (max, sum, o' = sum p C_V)
//     over its chunk of rows; the extra block does the same over the window
//     rows with the raw query;
//   - the last block of a unit to finish (atomic ticket, reset by that block)
//     merges the partials by log-sum-exp, applies B_V^T, adds the window part
//     and normalises. The output stays fp32 (the compute type).
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int MAXG = 8;  // query heads per kv head handled by one workgroup
constexpr int QS_FLOATS = (NT * MAXG > MAXG * D) ? NT * MAXG : MAXG * D;

__device__ __forceinline__ void unit_coords(const DecodeArgs &a, int ul, int &li, int &bi, int &h) {
  h = ul % a.L.kvh;
  const int t = ul / a.L.kvh;
  bi = t % a.L.batch;
  li = t / a.L.batch;
}

// block-wide max/sum of one value per head; red must hold 4 * MAXG floats
__device__ __forceinline__ void block_reduce_heads(float *vals, int g, float *red, bool is_max) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int hh = 0; hh < g; hh++) {
    float v = is_max ? max64(vals[hh]) : sum64(vals[hh]);
    if (l == 0) red[w * MAXG + hh] = v;
  }
  __syncthreads();
  for (int hh = 0; hh < g; hh++) {
    const float a0 = red[hh], a1 = red[MAXG + hh], a2 = red[2 * MAXG + hh], a3 = red[3 * MAXG + hh];
    vals[hh] = is_max ? fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)) : (a0 + a1) + (a2 + a3);
  }
  __syncthreads();
}

// log-sum-exp merge of a unit's chunk partials and window part; osm must
// hold MAXG * D floats of LDS
__device__ void merge_unit(const DecodeArgs &a, int ul, int u, float *osm) {
  __shared__ float wsc[MAXG][4];  // M, L, window factor
  int li, bi, h;
  unit_coords(a, ul, li, bi, h);
  const int g = a.L.g, rV = a.L.X[1].r, kV = a.kV;
  const int stride = 2 + rV;
  const float *part = a.L.part + (size_t)u * a.L.nchunk_max * g * stride;
  const float *wp = a.L.wpart + (size_t)u * g * (2 + D);
  const int tid = threadIdx.x;
  if (tid < g) {
    float M = wp[tid * (2 + D)];
    for (int c = 0; c < a.nchunk; c++) M = fmaxf(M, part[((size_t)c * g + tid) * stride]);
    float L = (wp[tid * (2 + D) + 1] > 0.f) ? wp[tid * (2 + D) + 1] * __expf(wp[tid * (2 + D)] - M) : 0.f;
    for (int c = 0; c < a.nchunk; c++) {
      const float lc = part[((size_t)c * g + tid) * stride + 1];
      if (lc > 0.f) L += lc * __expf(part[((size_t)c * g + tid) * stride] - M);
    }
    wsc[tid][0] = M;
    wsc[tid][1] = L;
    wsc[tid][2] = (wp[tid * (2 + D) + 1] > 0.f) ? __expf(wp[tid * (2 + D)] - M) : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < g * kV; idx += NT) {
    const int hh = idx / kV, j = idx - hh * kV;
    const float M = wsc[hh][0];
    float s = 0.f;
    for (int c = 0; c < a.nchunk; c++) {
      const float *pc = part + ((size_t)c * g + hh) * stride;
      if (pc[1] > 0.f) s += __expf(pc[0] - M) * pc[2 + j];
    }
    osm[hh * D + j] = s;
  }
  __syncthreads();
  const float *Bt = a.L.X[1].Bt + (size_t)u * rV * D;
  float *out = (float *)a.out + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
  for (int idx = tid; idx < g * D; idx += NT) {
    const int hh = idx / D, t = idx - hh * D;
    float s = 0.f;
    for (int j = 0; j < kV; j++) s += osm[hh * D + j] * Bt[(size_t)j * D + t];
    s += wsc[hh][2] * wp[hh * (2 + D) + 2 + t];
    out[idx] = s / wsc[hh][1];
  }
}

template <typename TC, typename TK>
__global__ void __launch_bounds__(NT) k_decode(const DecodeArgs a) {
  extern __shared__ float sm[];
  const int ul = blockIdx.y;
  const int u = a.u0 + ul;
  const int g = a.L.g;
  const int tid = threadIdx.x;
  float *red = sm;                 // 4 * MAXG
  float *qs = sm + 4 * MAXG;       // g x D (window) or g x kK (history); later nz x g x width
  float *ss = qs + QS_FLOATS;      // g x rows (rows <= chunk)
  const int ch = blockIdx.x;
  const bool window = (ch == a.nchunk);
  int rows, row0 = 0;
  if (window) {
    rows = a.e;
  } else {
    row0 = ch * a.L.chunk;
    rows = min(a.L.chunk, a.n - row0);
  }
  const int ldq = window ? D : a.kK;
  // query vectors
  if (window) {
    int li, bi, h;
    unit_coords(a, ul, li, bi, h);
    const TK *q = (const TK *)a.q + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
    for (int idx = tid; idx < g * D; idx += NT) qs[idx] = a.scale * ldf<TK>(q, idx);
  } else {
    // q' = scale * B_K^T q for the g heads of this kv head (16 lanes per dot)
    int li, bi, h;
    unit_coords(a, ul, li, bi, h);
    const TK *q = (const TK *)a.q + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
    const float *Bt = a.L.X[0].Bt + (size_t)u * a.L.X[0].r * D;
    const int lane = tid & 15, grp = tid >> 4;
    for (int pj = grp; pj < g * a.kK; pj += 16) {
      const int hh = pj / a.kK, jj = pj - hh * a.kK;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 8; t++)
        s += Bt[(size_t)jj * D + lane * 8 + t] * ldf<TK>(q, (size_t)hh * D + lane * 8 + t);
      s = sum16(s);
      if (lane == 0) qs[hh * a.kK + jj] = a.scale * s;
    }
  }
  __syncthreads();
  // scores: one thread per row
  float mx[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; hh++) mx[hh] = -INFINITY;
  if (window) {
    const TK *kr = (const TK *)a.L.X[0].ring + (size_t)u * a.L.rcap * D;
    for (int i = tid; i < rows; i += NT) {
      int pos = a.head + i;
      if (pos >= a.L.rcap) pos -= a.L.rcap;
      float s[MAXG];
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++) s[hh] = 0.f;
      for (int t = 0; t < D; t++) {
        const float x = ldf<TK>(kr, (size_t)pos * D + t);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) s[hh] += x * qs[hh * D + t];
      }
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++)
        if (hh < g) {
          ss[hh * a.L.chunk + i] = s[hh];
          mx[hh] = fmaxf(mx[hh], s[hh]);
        }
    }
  } else {
    const int rK = a.L.X[0].r;
    const TC *ck = (const TC *)a.L.X[0].C + (size_t)u * a.L.X[0].cstride + (size_t)row0 * rK;
    for (int i = tid; i < rows; i += NT) {
      float s[MAXG];
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++) s[hh] = 0.f;
      for (int j = 0; j < a.kK; j++) {
        const float x = ldf<TC>(ck, (size_t)i * rK + j);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) s[hh] += x * qs[hh * ldq + j];
      }
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++)
        if (hh < g) {
          ss[hh * a.L.chunk + i] = s[hh];
          mx[hh] = fmaxf(mx[hh], s[hh]);
        }
    }
  }
  block_reduce_heads(mx, g, red, true);
  float sum[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; hh++) sum[hh] = 0.f;
  for (int i = tid; i < rows; i += NT) {
#pragma unroll
    for (int hh = 0; hh < MAXG; hh++)
      if (hh < g) {
        const float pv = __expf(ss[hh * a.L.chunk + i] - mx[hh]);
        ss[hh * a.L.chunk + i] = pv;
        sum[hh] += pv;
      }
  }
  block_reduce_heads(sum, g, red, false);  // includes a barrier: ss is complete
  // weighted values: thread -> (column j, row slice z)
  const int width = window ? D : a.kV;
  const int nz = width > 0 ? NT / width : 0;
  float *acc_sm = qs;  // reuse: nz x g x width (<= NT * MAXG floats)
  float acc[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; hh++) acc[hh] = 0.f;
  const int j = width > 0 ? tid % width : 0;
  const int z = width > 0 ? tid / width : 0;
  if (width > 0 && z < nz) {
    if (window) {
      const TK *vr = (const TK *)a.L.X[1].ring + (size_t)u * a.L.rcap * D;
      for (int i = z; i < rows; i += nz) {
        int pos = a.head + i;
        if (pos >= a.L.rcap) pos -= a.L.rcap;
        const float x = ldf<TK>(vr, (size_t)pos * D + j);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) acc[hh] += ss[hh * a.L.chunk + i] * x;
      }
    } else {
      const int rV = a.L.X[1].r;
      const TC *cv = (const TC *)a.L.X[1].C + (size_t)u * a.L.X[1].cstride + (size_t)row0 * rV;
      for (int i = z; i < rows; i += nz) {
        const float x = ldf<TC>(cv, (size_t)i * rV + j);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) acc[hh] += ss[hh * a.L.chunk + i] * x;
      }
    }
  }
  __syncthreads();
  if (width > 0 && z < nz) {
#pragma unroll
    for (int hh = 0; hh < MAXG; hh++)
      if (hh < g) acc_sm[((size_t)z * g + hh) * width + j] = acc[hh];
  }
  __syncthreads();
  float *dst;
  int stride;
  if (window) {
    dst = a.L.wpart + (size_t)u * g * (2 + D);
    stride = 2 + D;
  } else {
    stride = 2 + a.L.X[1].r;
    dst = a.L.part + ((size_t)u * a.L.nchunk_max + ch) * g * stride;
  }
  for (int idx = tid; idx < g * width; idx += NT) {
    const int hh = idx / width, jj = idx - hh * width;
    float s = 0.f;
    for (int zz = 0; zz < nz; zz++) s += acc_sm[((size_t)zz * g + hh) * width + jj];
    dst[hh * stride + 2 + jj] = s;
  }
  if (tid < g) {
    dst[tid * stride + 0] = rows > 0 ? mx[tid] : -INFINITY;
    dst[tid * stride + 1] = rows > 0 ? sum[tid] : 0.f;
  }
  // ---- last block of the unit merges ------------------------------------
  __threadfence();  // this block's partial is visible device-wide before its ticket
  __syncthreads();
  int *flag = (int *)red;
  if (tid == 0) {
    const unsigned t = atomicAdd(a.L.ticket + u, 1u);
    flag[0] = (t == (unsigned)a.nchunk) ? 1 : 0;
  }
  __syncthreads();
  if (!flag[0]) return;
  __threadfence();
  merge_unit(a, ul, u, qs);
  if (tid == 0) a.L.ticket[u] = 0u;
}


// ===========================================================================
// bf16 storage: matrix-core decode (used when both ranks are multiples of 8)
//
// Each history wavefront takes a contiguous range of rows, in steps of 32
// rows, with v_mfma_f32_16x16x32_bf16:
//   scores   S (16 rows x 16 heads) = C_K tile (16 x 32 cols) . Q' (32 x 16)
//            A: 16 contiguous bytes of one C_K row per lane (coalesced);
//            B: q' in registers, split into bf16 hi + lo (about 16 bits).
//   values   o'^T (16 cols x 16 heads) += C_V^T (16 x 32 rows) . P^T (32 x 16)
//            The 32 K-slots of the step are ordered so that lane l's eight
//            softmax weights are exactly the eight scores its own output
//            fragments hold (rows 4q..4q+3 and 16+4q..16+4q+3, q = l/16);
//            P^T is then split hi + lo in registers, and the C_V^T fragment is
//            gathered from a per-wave LDS copy of the 32-row tile.
// Online softmax per wave (running max and sum per head); the waves of the
// unit's workgroup are then combined in LDS.
// ===========================================================================
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;


__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// two fp32 values to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// x = hi + lo with both parts bf16 (round to nearest even)
__device__ __forceinline__ void split8(const float *x, u32x4_t &hi, u32x4_t &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    h[i] = cvt_pk_bf16(x[2 * i], x[2 * i + 1]);
    l[i] = cvt_pk_bf16(x[2 * i] - __uint_as_float(h[i] << 16), x[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
  }
  hi = u32x4_t{h[0], h[1], h[2], h[3]};
  lo = u32x4_t{l[0], l[1], l[2], l[3]};
}

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__host__ __device__ __forceinline__ int tile_stride(int rsV) { return ((rsV + 15) / 16) * 16 + 4; }

// One 1024-thread workgroup per unit. Every wavefront streams a contiguous
// slice of the history rows (MFMA scores and values, online softmax, the
// next 32-row step's loads in flight while the current one is computed) and
// then a share of the window rows (16 lanes per 128-wide row); the partials
// of all waves are combined in LDS and the workgroup writes the unit's
// outputs. No workgroup talks to another, so no device-scope fence is needed
// (on a multi-XCD part each one writes back and invalidates the XCD's L2).
constexpr int NTU = 1024;
constexpr int NWU = NTU / 64;
constexpr int WH = 2;  // window heads per pass (register budget: 128 VGPRs per lane)

// LDS in floats: q' and its fragments, then the per-wave tiles (history) or
// the combine scratch, then (optionally) the window rows, K then V, bf16.
__host__ __device__ inline size_t decode_unit_qs(int rsK) {
  return (size_t)MAXG * (rsK > 0 ? rsK : 1) + 4 * 64 * 2 * 4 + 4 * 64 * 4;  // q', its fragments, q fragments
}
// nwo = waves that leave window partials: all of them on the ring path, one
// per 32-row window step when the window is staged
__host__ __device__ inline size_t decode_unit_big(int rsV, int g, int nwo) {
  const size_t tiles = (size_t)NWU * 32 * tile_stride(rsV) * 2 / 4;
  const size_t comb = 2 * (size_t)NWU * MAXG + (size_t)NWU * g * rsV + (size_t)nwo * g * (2 + D) +
                      (size_t)g * rsV + (size_t)g * D + 8 * MAXG;
  return tiles > comb ? tiles : comb;
}
__host__ __device__ inline int decode_unit_nwo(int ewin) {
  const int s = (ewin + 31) / 32;
  return (ewin > 0 && s < NWU) ? s : NWU;
}
// staged window rows are padded to WSTR bf16 (272 bytes): 16 lanes reading 16
// consecutive rows then fall into distinct banks
constexpr int WSTR = D + 8;
// ewin = staged window rows (0: window read from the ring)
__host__ __device__ inline size_t decode_unit_lds(int rsK, int rsV, int g, int ewin) {
  return sizeof(float) *
         (decode_unit_qs(rsK) + decode_unit_big(rsV, g, decode_unit_nwo(ewin)) + (size_t)ewin * WSTR);
}

// Window rows of the workgroup's window share: from the LDS copy or the ring.
template <bool STAGED>
__device__ __forceinline__ const uint16_t *win_row(const uint16_t *base, int i, int head, int rcap) {
  if (STAGED) return base + (size_t)i * D;
  int pos = head + i;
  if (pos >= rcap) pos -= rcap;
  return base + (size_t)pos * D;
}

template <int KS, int NTV>
__device__ __forceinline__ void load_step(const uint16_t *CK, const uint16_t *CV, int rsK, int rsV, int rb,
                                          int we, int lane, u32x4_t *ka, u32x4_t *kb, u32x4_t *vv) {
  const int hq = lane & 15, qd = lane >> 4;
  const int cpr = rsV / 8;
#pragma unroll
  for (int kc = 0; kc < KS; kc++) {
    const int col = kc * 32 + 8 * qd;
    const int r0 = rb + hq, r1 = rb + 16 + hq;
    ka[kc] = u32x4_t{0u, 0u, 0u, 0u};
    kb[kc] = u32x4_t{0u, 0u, 0u, 0u};
    if (col < rsK) {
      if (r0 < we) ka[kc] = *(const u32x4_t *)(CK + (size_t)r0 * rsK + col);
      if (r1 < we) kb[kc] = *(const u32x4_t *)(CK + (size_t)r1 * rsK + col);
    }
  }
  // the 32-row C_V tile: 32 x rsV/8 chunks of 16 bytes; 64 * NTV >= 4 * rsV covers them all
#pragma unroll
  for (int z = 0; z < NTV; z++) {
    const int idx = lane + 64 * z;
    const int rr = idx / cpr, c8 = idx - rr * cpr;
    vv[z] = u32x4_t{0u, 0u, 0u, 0u};
    if (idx < 32 * cpr && rb + rr < we) vv[z] = *(const u32x4_t *)(CV + (size_t)(rb + rr) * rsV + c8 * 8);
  }
}

template <int NTV>
__device__ __forceinline__ void store_tile(uint16_t *tile, int ts, int rsV, int lane, const u32x4_t *vv) {
  const int cpr = rsV / 8;
#pragma unroll
  for (int z = 0; z < NTV; z++) {
    const int idx = lane + 64 * z;
    const int rr = idx / cpr, c8 = idx - rr * cpr;
    if (idx < 32 * cpr) {
      uint2 *dstp = (uint2 *)(tile + rr * ts + c8 * 8);
      dstp[0] = uint2{vv[z][0], vv[z][1]};
      dstp[1] = uint2{vv[z][2], vv[z][3]};
    }
  }
}

// int8 storage: the same step over codes of U. The K order of the score
// products is permuted so that lane l loads 16 contiguous codes of its rows
// rb + l % 16 and rb + 16 + l % 16, columns 64 p + 16 (l / 16) .. +15 for each
// whole pair p of K steps (step kc takes the half kc % 2 of pair kc / 2); a
// last unpaired step (KS odd) loads 8 codes, columns 32 kc + 8 (l / 16) .. +7.
// The q' fragments follow the same order. The 32-row C_V tile is 32 rsV contiguous
// bytes read in 16-byte pieces, and each lane takes the scales of the 8 rows
// its score fragments hold (rows rb + 4 (l / 16) + i and rb + 16 + 4 (l / 16)
// + i); rows at or past `we` get scale 0.
__device__ __forceinline__ u32x4_t load16_i8(const uint8_t *p, bool al16) {
  if (al16) return *(const u32x4_t *)p;
  const uint2 lo = *(const uint2 *)p, hi = *(const uint2 *)(p + 8);  // 8-byte aligned rows
  return u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

template <int KS, int NV>
__device__ __forceinline__ void load_step_i8(const uint8_t *CK, const uint8_t *CV, const float *sK,
                                             const float *sV, int rsK, int rsV, int rb, int we, int lane,
                                             u32x4_t *ka, u32x4_t *kb, u32x4_t *vv, float *fk, float *fv) {
  const int hq = lane & 15, qd = lane >> 4;
  const bool al16 = (rsK & 15) == 0;
  constexpr int KP = (KS + 1) / 2;
#pragma unroll
  for (int p = 0; p < KP; p++) {
    // a 16-code piece that starts below column rsK may end past it (rsK % 16
    // == 8): the next row's codes then meet zero entries of q'
    const bool single = 2 * p + 1 == KS;
    const int col = single ? p * 64 + 8 * qd : p * 64 + 16 * qd;
    const int r0 = rb + hq, r1 = rb + 16 + hq;
    ka[p] = u32x4_t{0u, 0u, 0u, 0u};
    kb[p] = u32x4_t{0u, 0u, 0u, 0u};
    if (col < rsK) {
      if (single) {
        if (r0 < we) {
          const uint2 v = *(const uint2 *)(CK + (size_t)r0 * rsK + col);
          ka[p] = u32x4_t{v.x, v.y, 0u, 0u};
        }
        if (r1 < we) {
          const uint2 v = *(const uint2 *)(CK + (size_t)r1 * rsK + col);
          kb[p] = u32x4_t{v.x, v.y, 0u, 0u};
        }
      } else {
        if (r0 < we) ka[p] = load16_i8(CK + (size_t)r0 * rsK + col, al16);
        if (r1 < we) kb[p] = load16_i8(CK + (size_t)r1 * rsK + col, al16);
      }
    }
  }
#pragma unroll
  for (int z = 0; z < NV; z++) {
    const int idx = lane + 64 * z;
    vv[z] = u32x4_t{0u, 0u, 0u, 0u};
    // a piece's first byte decides the load; its second half may reach row
    // we, which is still inside the unit's rows or its 256-byte pad
    if (idx < 2 * rsV && rb + (16 * idx) / rsV < we)
      vv[z] = *(const u32x4_t *)(CV + (size_t)rb * rsV + 16 * idx);
  }
  // rows rb + 4 qd .. +3 and rb + 16 + 4 qd .. +3: one aligned 16-byte piece
  // each (rb and the per-unit scale stride are multiples of 4)
#pragma unroll
  for (int hf = 0; hf < 2; hf++) {
    const int row = rb + 16 * hf + 4 * qd;
    f32x4_t a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (row < we) {
      a = *(const f32x4_t *)(sK + row);
      b = *(const f32x4_t *)(sV + row);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      fk[4 * hf + i] = row + i < we ? a[i] : 0.f;
      fv[4 * hf + i] = row + i < we ? b[i] : 0.f;
    }
  }
}

// the 16-byte pieces of the C_V tile as bf16 into the wave's LDS tile; each
// 8-code half goes to its own row (rows past we as zeros)
template <int NV>
__device__ __forceinline__ void store_tile_i8(uint16_t *tile, int ts, int rsV, int rb, int we, int lane,
                                              const u32x4_t *vv) {
#pragma unroll
  for (int z = 0; z < NV; z++) {
    const int idx = lane + 64 * z;
    if (idx < 2 * rsV) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int off = 16 * idx + 8 * h;
        const int rr = off / rsV, c = off - rr * rsV;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (rb + rr < we) i8x8_bf16(vv[z][2 * h], vv[z][2 * h + 1], w);
        uint2 *dstp = (uint2 *)(tile + rr * ts + c);
        dstp[0] = uint2{w[0], w[1]};
        dstp[1] = uint2{w[2], w[3]};
      }
    }
  }
}

// The matrix-core decode keeps its scores in base-2 units (scale * log2(e)
// folded into q' and the window scores), so every softmax weight, rescale
// and merge factor is one v_exp_f32.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Window rows of one unit straight from the ring (used when the window does
// not fit in LDS): row i goes to lane group (i mod 64) of the workgroup (16
// lanes per 128-wide row), WH heads per pass, online softmax; the 4 lane
// groups of a wave are combined with shuffles and each wave leaves (max, sum,
// values) per head in wo.
__device__ __forceinline__ void window_part(const DecodeArgs &a, const uint16_t *q, const uint16_t *kr,
                                            const uint16_t *vr, float *wo, int g, int wv, int lane) {
  const int l16 = lane & 15, grp = lane >> 4;
  const int gg = wv * 4 + grp;
  for (int h0 = 0; h0 < g; h0 += WH) {
    float qv[WH][8], wa[WH][8], wm[WH], wl[WH];
#pragma unroll
    for (int j = 0; j < WH; j++) {
      wm[j] = -INFINITY;
      wl[j] = 0.f;
#pragma unroll
      for (int t = 0; t < 8; t++) {
        wa[j][t] = 0.f;
        qv[j][t] = (h0 + j < g) ? a.scale * LOG2E * bf2f(q[(size_t)(h0 + j) * D + l16 * 8 + t]) : 0.f;
      }
    }
    for (int i = gg; i < a.e; i += 4 * NWU) {
      const u32x4_t kw = *(const u32x4_t *)(win_row<false>(kr, i, a.head, a.L.rcap) + l16 * 8);
      const u32x4_t vw = *(const u32x4_t *)(win_row<false>(vr, i, a.head, a.L.rcap) + l16 * 8);
      float kx[8], vx[8];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        kx[2 * t] = __uint_as_float(kw[t] << 16);
        kx[2 * t + 1] = __uint_as_float(kw[t] & 0xffff0000u);
        vx[2 * t] = __uint_as_float(vw[t] << 16);
        vx[2 * t + 1] = __uint_as_float(vw[t] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < WH; j++) {
        float sc = 0.f;
#pragma unroll
        for (int t = 0; t < 8; t++) sc += kx[t] * qv[j][t];
        sc = sum16(sc);
        const float mn = fmaxf(wm[j], sc);
        const float al = ex2(wm[j] - mn);
        const float pv = ex2(sc - mn);
        wl[j] = wl[j] * al + pv;
#pragma unroll
        for (int t = 0; t < 8; t++) wa[j][t] = wa[j][t] * al + pv * vx[t];
        wm[j] = mn;
      }
    }
    // combine the 4 lane groups of the wave (xor 16, 32)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
      for (int j = 0; j < WH; j++) {
        const float mo = __shfl_xor(wm[j], off);
        const float lo = __shfl_xor(wl[j], off);
        const float mn = fmaxf(wm[j], mo);
        const float ms = (mn == -INFINITY) ? 0.f : mn;
        const float f0 = ex2(wm[j] - ms), f1 = ex2(mo - ms);
        wl[j] = wl[j] * f0 + lo * f1;
#pragma unroll
        for (int t = 0; t < 8; t++) {
          const float ao = __shfl_xor(wa[j][t], off);
          wa[j][t] = wa[j][t] * f0 + ao * f1;
        }
        wm[j] = mn;
      }
    }
    if (grp == 0) {
#pragma unroll
      for (int j = 0; j < WH; j++) {
        if (h0 + j < g) {
          float *w = wo + ((size_t)wv * g + h0 + j) * (2 + D);
          if (l16 == 0) {
            w[0] = wm[j];
            w[1] = wl[j];
          }
#pragma unroll
          for (int t = 0; t < 8; t++) w[2 + l16 * 8 + t] = wa[j][t];
        }
      }
    }
  }
}

// Window rows staged in LDS, on matrix cores: the window is one more
// history-like stream with 128 key dims (4 K steps, B = q itself, exact in
// bf16, the scale applied to the fp32 scores) and 128 value columns (8 tiles).
// Wave wv takes the 32-row steps wv, wv + NWU, ...; every wave leaves its
// (max, sum, values) per head in wo[wv].
__device__ __forceinline__ void window_mfma(const DecodeArgs &a, int e, const u32x4_t *qfrag, const uint16_t *wk,
                                            const uint16_t *wvr, float *wo, int g, int wv, int lane) {
  const int hq = lane & 15, qd = lane >> 4;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; nt++) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int rb = 32 * wv; rb < e; rb += 32 * NWU) {
    f32x4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
    const int r0 = rb + hq, r1 = rb + 16 + hq;
#pragma unroll
    for (int kc = 0; kc < 4; kc++) {
      const int col = kc * 32 + 8 * qd;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      const u32x4_t k0 = (r0 < e) ? *(const u32x4_t *)(wk + (size_t)r0 * WSTR + col) : z;
      const u32x4_t k1 = (r1 < e) ? *(const u32x4_t *)(wk + (size_t)r1 * WSTR + col) : z;
      const u32x4_t bq = qfrag[kc * 64 + lane];
      d0 = mfma16(k0, bq, d0);
      d1 = mfma16(k1, bq, d1);
    }
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      s[i] = (rb + 4 * qd + i < e) ? (a.scale * LOG2E) * d0[i] : -INFINITY;
      s[4 + i] = (rb + 16 + 4 * qd + i < e) ? (a.scale * LOG2E) * d1[i] : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    const float al = ex2(m - ms);
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      p[i] = ex2(s[i] - ms);
      ps += p[i];
    }
    l = l * al + ps;
    m = mn;
    u32x4_t phi, plo;
    split8(p, phi, plo);
#pragma unroll
    for (int nt = 0; nt < 8; nt++) {
      acc[nt] *= al;
      const int col = nt * 16 + hq;
      uint16_t v8[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int row = rb + ((i < 4) ? (4 * qd + i) : (16 + 4 * qd + i - 4));
        v8[i] = (row < e) ? wvr[(size_t)row * WSTR + col] : (uint16_t)0;
      }
      const u32x4_t av = {pack2(v8[0], v8[1]), pack2(v8[2], v8[3]), pack2(v8[4], v8[5]), pack2(v8[6], v8[7])};
      acc[nt] = mfma16(av, phi, acc[nt]);
      acc[nt] = mfma16(av, plo, acc[nt]);
    }
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (hq < g && 32 * wv < e) {  // waves with window steps: the first decode_unit_nwo(e)
    float *w = wo + ((size_t)wv * g + hq) * (2 + D);
    if (qd == 0) {
      w[0] = m;
      w[1] = l;
    }
#pragma unroll
    for (int nt = 0; nt < 8; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) w[2 + nt * 16 + 4 * qd + i] = acc[nt][i];
  }
}

// SPLIT: grid (units, nsplit); workgroup s takes history rows
// [s split_rows, (s + 1) split_rows) and workgroup 0 also the window; each
// leaves its partial (max, sum, o', window values) per query head in
// a.spart for k_decode_merge instead of writing the output.
// I8: int8 storage of U with per-row scales (scores C_K q' = U_K (Sigma_K q'),
// values p^T C_V = (p^T U_V) Sigma_V, each row's scale on its score and its
// softmax weight).
template <int KS, int NTV, bool SPLIT, bool I8>
__global__ void __launch_bounds__(NTU) k_decode_unit(const DecodeArgs a) {
  extern __shared__ float sm[];
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int g = a.L.g, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rsK = a.L.X[0].r, rsV = a.L.X[1].r;
  const bool hasw = !SPLIT || blockIdx.y == 0;  // this workgroup attends the window
  float *qsm = sm;                                          // g x rsK: q'
  u32x4_t *frag = (u32x4_t *)(qsm + (size_t)MAXG * rsK);    // [(kc*2 + part)*64 + lane]
  u32x4_t *qfrag = frag + 4 * 2 * 64;                        // [kc*64 + lane]: q itself (bf16)
  float *big = qsm + decode_unit_qs(rsK);                   // tiles, then combine scratch
  const int nwo = hasw ? decode_unit_nwo(a.wlds ? a.e + a.nnew : 0) : 0;
  uint16_t *wsm = (uint16_t *)(big + decode_unit_big(rsV, g, nwo));  // [2][e][WSTR] window copy
  int li, bi, h;
  unit_coords(a, ul, li, bi, h);
  const uint16_t *q = (const uint16_t *)a.q + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
  const uint16_t *kr = (const uint16_t *)a.L.X[0].ring + (size_t)u * a.L.rcap * D;
  const uint16_t *vr = (const uint16_t *)a.L.X[1].ring + (size_t)u * a.L.rcap * D;
  // The window rows are copied to LDS in batches of WB 16-byte chunks per
  // thread; the first batch's loads are in flight during the q' projection.
  constexpr int WB = 8;
  const int ew = hasw ? a.e + a.nnew : 0;          // window rows, the appended one last
  const int wch = a.wlds ? 2 * ew * (D / 8) : 0;  // K rows, then V rows
  const size_t nrow_off = (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.kvh + h) * D;
  u32x4_t wbuf[WB];
  auto win_load = [&](int c0) {
#pragma unroll
    for (int z = 0; z < WB; z++) {
      const int c = c0 + z * NTU + tid;
      wbuf[z] = u32x4_t{0u, 0u, 0u, 0u};
      if (c < wch) {
        const int which = c >= ew * (D / 8);
        const int rem = c - which * ew * (D / 8);
        const int i = rem >> 4, part = rem & 15;
        const uint16_t *src = (i < a.e) ? win_row<false>(which ? vr : kr, i, a.head, a.L.rcap)
                                        : (const uint16_t *)(which ? a.nv : a.nk) + nrow_off;
        wbuf[z] = *(const u32x4_t *)(src + part * 8);
      }
    }
  };
  auto win_store = [&](int c0) {
#pragma unroll
    for (int z = 0; z < WB; z++) {
      const int c = c0 + z * NTU + tid;
      if (c < wch) {
        const int which = c >= ew * (D / 8);
        const int rem = c - which * ew * (D / 8);
        const int i = rem >> 4, part = rem & 15;
        *(u32x4_t *)(wsm + ((size_t)which * ew + i) * WSTR + part * 8) = wbuf[z];
        if (i >= a.e) {  // the appended row also enters the ring
          uint16_t *ring = (uint16_t *)(which ? a.L.X[1].ring : a.L.X[0].ring) + (size_t)u * a.L.rcap * D;
          *(u32x4_t *)((uint16_t *)win_row<false>(ring, i, a.head, a.L.rcap) + part * 8) = wbuf[z];
        }
      }
    }
  };
  if (wch > 0) win_load(0);
  // this wave's history slice; its first step is loaded before the projection
  const int h0 = SPLIT ? blockIdx.y * a.split_rows : 0;
  const int h1 = SPLIT ? min(a.n, h0 + a.split_rows) : a.n;
  int per = (max(h1 - h0, 0) + NWU - 1) / NWU;
  per = ((per + 31) / 32) * 32;
  const int wb = h0 + wv * per;
  const int we = min(h1, wb + per);
  const uint16_t *CK = (const uint16_t *)a.L.X[0].C + (size_t)u * a.L.X[0].cstride;
  const uint16_t *CV = (const uint16_t *)a.L.X[1].C + (size_t)u * a.L.X[1].cstride;
  const uint8_t *CK8 = (const uint8_t *)a.L.X[0].C + (size_t)u * a.L.X[0].cstride;
  const uint8_t *CV8 = (const uint8_t *)a.L.X[1].C + (size_t)u * a.L.X[1].cstride;
  const float *sK = I8 ? a.L.X[0].cs + (size_t)u * cs_stride(a.L.ncap) : nullptr;
  const float *sV = I8 ? a.L.X[1].cs + (size_t)u * cs_stride(a.L.ncap) : nullptr;
  // prefetching the next step doubles the load registers: only when they fit
  constexpr int NV = I8 ? (NTV + 1) / 2 : NTV;  // 16-byte pieces of the C_V tile per lane
  constexpr bool PF = I8 ? (NV + KS) <= 2 : (NTV + 2 * KS) <= 6;  // int8: 8 row scales per kind too
  // int8 at small ranks: 64-row steps of two loaded halves instead of a
  // prefetched 32-row step (measured: 8-10% faster there; no gain for bf16)
  constexpr bool TWO = I8 && PF && KS == 1;
  constexpr int KP = (KS + 1) / 2;  // int8: K-step pairs of 16-byte code pieces
  u32x4_t ka[KS], kb[KS], vv[NV];
  u32x4_t ka8[KP], kb8[KP];
  float fk[8], fv[8];
  auto load = [&](int rb, u32x4_t *ka_, u32x4_t *kb_, u32x4_t *ka8_, u32x4_t *kb8_, u32x4_t *vv_, float *fk_,
                  float *fv_) {
    if constexpr (I8)
      load_step_i8<KS, NV>(CK8, CV8, sK, sV, rsK, rsV, rb, we, lane, ka8_, kb8_, vv_, fk_, fv_);
    else
      load_step<KS, NTV>(CK, CV, rsK, rsV, rb, we, lane, ka_, kb_, vv_);
  };
  if (PF && wb < we) load(wb, ka, kb, ka8, kb8, vv, fk, fv);
  // q' = scale * log2(e) * B_K^T q, zero beyond the current rank (16 lanes per dot)
  {
    const float *Bt = a.L.X[0].Bt + (size_t)u * rsK * D;
    const int l16 = tid & 15, grp = tid >> 4;
    for (int pj = grp; pj < g * rsK; pj += NTU / 16) {
      const int hh = pj / rsK, jj = pj - hh * rsK;
      float s = 0.f;
      if (jj < a.kK) {
#pragma unroll
        for (int t = 0; t < 8; t++) s += Bt[(size_t)jj * D + l16 * 8 + t] * bf2f(q[(size_t)hh * D + l16 * 8 + t]);
      }
      s = sum16(s);
      if constexpr (I8) s *= (jj < a.kK) ? a.L.X[0].sig[(size_t)u * rsK + jj] : 0.f;  // Sigma_K q'
      if (l16 == 0) qsm[hh * rsK + jj] = (a.scale * LOG2E) * s;
    }
  }
  if (a.wlds && tid < 4 * 64) {
    // B fragments of q for the window scores: head l % 16, dims 32 kc + 8 (l / 16) .. +7
    const int kc = tid >> 6, ln = tid & 63, fq = ln & 15;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (fq < g) v = *(const u32x4_t *)(q + (size_t)fq * D + kc * 32 + 8 * (ln >> 4));
    qfrag[kc * 64 + ln] = v;
  }
  if (wch > 0) {
    win_store(0);
    for (int c0 = WB * NTU; c0 < wch; c0 += WB * NTU) {
      win_load(c0);
      win_store(c0);
    }
  }
  __syncthreads();
  // MFMA B fragments of q' (bf16 hi and lo) per lane, shared by all waves
  if (tid < 64 * KS) {
    const int kc = tid >> 6, ln = tid & 63;
    const int fq = ln & 15, fd = ln >> 4;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      // int8 storage permutes the K order of whole step pairs (see load_step_i8)
      const int col = (I8 && (kc | 1) < KS) ? 64 * (kc >> 1) + 16 * fd + 8 * (kc & 1) + i : kc * 32 + 8 * fd + i;
      x[i] = (fq < g && col < rsK) ? qsm[fq * rsK + col] : 0.f;
    }
    split8(x, frag[(kc * 2) * 64 + ln], frag[(kc * 2 + 1) * 64 + ln]);
  }
  __syncthreads();
  const int hq = lane & 15, qd = lane >> 4;
  // ---- history rows of this wave ----------------------------------------
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[NTV];
#pragma unroll
  for (int nt = 0; nt < NTV; nt++) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    const int ts = tile_stride(rsV);
    uint16_t *tile = (uint16_t *)big + (size_t)wv * 32 * ts;
    auto put_tile = [&](int rb, const u32x4_t *vv_) {
      if constexpr (I8)
        store_tile_i8<NV>(tile, ts, rsV, rb, we, lane, vv_);
      else
        store_tile<NTV>(tile, ts, rsV, lane, vv_);
    };
    // one 32-row step over registers loaded by `load` (its C_V tile already in
    // the wave's LDS tile): scores, online softmax, weighted values
    auto compute = [&](int rb, u32x4_t *ka, u32x4_t *kb, const u32x4_t *ka8, const u32x4_t *kb8, const float *fk,
                       const float *fv) {
        if constexpr (I8) {
#pragma unroll
          for (int kc = 0; kc < KS; kc++) {
            const int pp = kc >> 1, hh = 2 * (kc & 1);
            uint32_t w[4];
            i8x8_bf16(ka8[pp][hh], ka8[pp][hh + 1], w);
            ka[kc] = u32x4_t{w[0], w[1], w[2], w[3]};
            i8x8_bf16(kb8[pp][hh], kb8[pp][hh + 1], w);
            kb[kc] = u32x4_t{w[0], w[1], w[2], w[3]};
          }
        }
        f32x4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KS; kc++) {
          const u32x4_t bh = frag[(kc * 2) * 64 + lane], bl = frag[(kc * 2 + 1) * 64 + lane];
          d0 = mfma16(ka[kc], bh, d0);
          d0 = mfma16(ka[kc], bl, d0);
          d1 = mfma16(kb[kc], bh, d1);
          d1 = mfma16(kb[kc], bl, d1);
        }
        float s[8];
        if (rb + 32 <= we) {  // a whole step (all but a wave's last): no row past we
#pragma unroll
          for (int i = 0; i < 4; i++) {
            // int8 storage: each row's score takes its scale
            s[i] = I8 ? d0[i] * fk[i] : d0[i];
            s[4 + i] = I8 ? d1[i] * fk[4 + i] : d1[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float f0 = I8 ? fk[i] : 1.f, f1 = I8 ? fk[4 + i] : 1.f;
            s[i] = (rb + 4 * qd + i < we) ? d0[i] * f0 : -INFINITY;
            s[4 + i] = (rb + 16 + 4 * qd + i < we) ? d1[i] * f1 : -INFINITY;
          }
        }
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 8; i++) mx = fmaxf(mx, s[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float ms = (mn == -INFINITY) ? 0.f : mn;
        const float al = ex2(m - ms);
        float p[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          p[i] = ex2(s[i] - ms);
          ps += p[i];
        }
        l = l * al + ps;
        m = mn;
#pragma unroll
        for (int nt = 0; nt < NTV; nt++) acc[nt] *= al;
        u32x4_t phi, plo;
        if constexpr (I8) {
          float pv[8];
#pragma unroll
          for (int i = 0; i < 8; i++) pv[i] = p[i] * fv[i];
          split8(pv, phi, plo);
        } else {
          split8(p, phi, plo);
        }
#pragma unroll
        for (int nt = 0; nt < NTV; nt++) {
          const int col = nt * 16 + hq;
          uint16_t v8[8];
#pragma unroll
          for (int i = 0; i < 8; i++) {
            const int row = (i < 4) ? (4 * qd + i) : (16 + 4 * qd + i - 4);
            v8[i] = (col < rsV) ? tile[row * ts + col] : (uint16_t)0;
          }
          const u32x4_t av = {pack2(v8[0], v8[1]), pack2(v8[2], v8[3]), pack2(v8[4], v8[5]), pack2(v8[6], v8[7])};
          acc[nt] = mfma16(av, phi, acc[nt]);
          acc[nt] = mfma16(av, plo, acc[nt]);
        }
    };
    if (wb < we) {
      if constexpr (TWO) {
        // small ranks: both halves of a 64-row step are loaded at once, so one
        // memory latency serves 64 rows (the second half's loads are issued
        // even when it is empty: every lane's rows are then past we and masked)
        for (int rb = wb; rb < we; rb += 64) {
          u32x4_t nka[KS], nkb[KS], nvv[NV];
          u32x4_t nka8[KP], nkb8[KP];
          float nfk[8], nfv[8];
          load(rb, ka, kb, ka8, kb8, vv, fk, fv);
          load(rb + 32, nka, nkb, nka8, nkb8, nvv, nfk, nfv);
          put_tile(rb, vv);
          wave_fence();
          compute(rb, ka, kb, ka8, kb8, fk, fv);
          wave_fence();
          if (rb + 32 < we) {
            put_tile(rb + 32, nvv);
            wave_fence();
            compute(rb + 32, nka, nkb, nka8, nkb8, nfk, nfv);
            wave_fence();
          }
        }
      } else {
      if constexpr (PF) {
        put_tile(wb, vv);
        wave_fence();
      }
      for (int rb = wb; rb < we; rb += 32) {
        const bool more = rb + 32 < we;
        u32x4_t nka[KS], nkb[KS], nvv[NV];
        u32x4_t nka8[KP], nkb8[KP];
        float nfk[8], nfv[8];
        if constexpr (PF) {
          if (more) load(rb + 32, nka, nkb, nka8, nkb8, nvv, nfk, nfv);
        } else {
          load(rb, ka, kb, ka8, kb8, vv, fk, fv);
          put_tile(rb, vv);
          wave_fence();
        }
        compute(rb, ka, kb, ka8, kb8, fk, fv);
        wave_fence();
        if constexpr (PF) {
          if (more) {
            put_tile(rb + 32, nvv);
#pragma unroll
            for (int kc = 0; kc < KS; kc++) {
              ka[kc] = nka[kc];
              kb[kc] = nkb[kc];
            }
#pragma unroll
            for (int pp = 0; pp < KP; pp++) {
              ka8[pp] = nka8[pp];
              kb8[pp] = nkb8[pp];
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
              fk[i] = nfk[i];
              fv[i] = nfv[i];
            }
          }
          wave_fence();
        }
      }
      }
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
    }
  }
  __syncthreads();  // tiles are free from here on
  // B_V for the output projection, loaded now so that the window and combine
  // phases hide the latency: output element (hh, t) is split over jsplit
  // adjacent lanes, lane part jp holding B_V[j][t] for j = jp, jp + jsplit, ...
  const int jsplit = (g * D >= NTU) ? 1 : NTU / (g * D);  // 1, 2, 4 or 8
  const bool bv_early = rsV <= 16 * jsplit && g * D <= NTU;
  const int ot = tid / jsplit, jp = tid - ot * jsplit;
  const float *Bv = a.L.X[1].Bt + (size_t)u * rsV * D;
  float bvr[16];
  if (bv_early) {
#pragma unroll
    for (int z = 0; z < 16; z++) {
      const int j = jp + jsplit * z;
      bvr[z] = (ot < g * D && j < a.kV) ? Bv[(size_t)j * D + (ot & (D - 1))] : 0.f;
    }
  }
  float *hm = big;                                  // [NWU][MAXG] max
  float *hl = hm + NWU * MAXG;                      // [NWU][MAXG] sum
  float *ha = hl + NWU * MAXG;                      // [NWU][g][rsV] o'
  float *wo = ha + (size_t)NWU * g * rsV;           // [nwo][g][2 + D] window (m, l, o)
  float *op = wo + (size_t)nwo * g * (2 + D);       // [g][rsV] merged o'
  float *ow = op + (size_t)g * rsV;                 // [g][D] merged window values
  float *fac = ow + (size_t)g * D;                  // [MAXG][8]: shift, L
  if (hq < g) {
    if (qd == 0) {
      hm[wv * MAXG + hq] = m;
      hl[wv * MAXG + hq] = l;
    }
    const float *sgV = a.L.X[1].sig + (size_t)u * rsV;
#pragma unroll
    for (int nt = 0; nt < NTV; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int col = nt * 16 + 4 * qd + i;
        // int8 storage holds U_V: o' = (p^T U_V) Sigma_V
        if (col < rsV) ha[((size_t)wv * g + hq) * rsV + col] = I8 ? acc[nt][i] * sgV[col] : acc[nt][i];
      }
  }
  // ---- window rows: row i goes to lane group (i mod 64) of the workgroup ----
  if (hasw) {
    if (a.wlds)
      window_mfma(a, ew, qfrag, wsm, wsm + (size_t)ew * WSTR, wo, g, wv, lane);
    else
      window_part(a, q, kr, vr, wo, g, wv, lane);
  }
  __syncthreads();
  // ---- combine all waves: per head the max, the sum, o' and window values ---
  if (tid < g) {
    float M = -INFINITY;
    for (int w = 0; w < NWU; w++) M = fmaxf(M, hm[w * MAXG + tid]);
    for (int w = 0; w < nwo; w++) M = fmaxf(M, wo[((size_t)w * g + tid) * (2 + D)]);
    const float ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    for (int w = 0; w < NWU; w++) L += ex2(hm[w * MAXG + tid] - ms) * hl[w * MAXG + tid];
    for (int w = 0; w < nwo; w++) {
      const float *ww = wo + ((size_t)w * g + tid) * (2 + D);
      L += ex2(ww[0] - ms) * ww[1];
    }
    fac[tid * 8 + 0] = ms;
    fac[tid * 8 + 1] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < g * rsV; idx += NTU) {
    const int hh = idx / rsV, j = idx - hh * rsV;
    const float ms = fac[hh * 8];
    float s = 0.f;
    for (int w = 0; w < NWU; w++) s += ex2(hm[w * MAXG + hh] - ms) * ha[((size_t)w * g + hh) * rsV + j];
    op[idx] = s;
  }
  for (int idx = tid; idx < g * D; idx += NTU) {
    const int hh = idx / D, t = idx - hh * D;
    const float ms = fac[hh * 8];
    float s = 0.f;
    for (int w = 0; w < nwo; w++) {
      const float *ww = wo + ((size_t)w * g + hh) * (2 + D);
      s += ex2(ww[0] - ms) * ww[2 + t];
    }
    ow[idx] = s;
  }
  __syncthreads();
  if constexpr (SPLIT) {
    // partial of this workgroup: (max, sum, o', window values) per head
    const int rs = 2 + rsV + D;
    float *rec = a.spart + ((size_t)ul * gridDim.y + blockIdx.y) * g * rs;
    for (int idx = tid; idx < g * rs; idx += NTU) {
      const int hh = idx / rs, t = idx - hh * rs;
      const float L = fac[hh * 8 + 1];
      float v;
      if (t == 0)
        v = (L > 0.f) ? fac[hh * 8] : -INFINITY;
      else if (t == 1)
        v = L;
      else if (t < 2 + rsV)
        v = op[hh * rsV + t - 2];
      else
        v = ow[hh * D + t - 2 - rsV];
      rec[idx] = v;
    }
    return;
  }
  float *out = (float *)a.out + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
  if (bv_early) {
    const int hh = ot / D;
    float s = 0.f;
    if (ot < g * D) {
#pragma unroll
      for (int z = 0; z < 16; z++) {
        const int j = jp + jsplit * z;
        if (j < rsV) s += op[hh * rsV + j] * bvr[z];
      }
    }
    for (int off = 1; off < jsplit; off <<= 1) s += __shfl_xor(s, off);
    if (ot < g * D && jp == 0) out[ot] = (ow[ot] + s) / fac[hh * 8 + 1];
  } else {
    for (int idx = tid; idx < g * D; idx += NTU) {
      const int hh = idx / D, t = idx - hh * D;
      float s = ow[idx];
      for (int j = 0; j < a.kV; j++) s += op[hh * rsV + j] * Bv[(size_t)j * D + t];
      out[idx] = s / fac[hh * 8 + 1];
    }
  }
}

// Log-sum-exp merge of the split partials of k_decode_unit<..., true>: per
// query head M = max_s m_s, L = sum_s l_s e^(m_s - M), then
// out = (sum_s e^(m_s - M) w_s + (sum_s e^(m_s - M) o'_s) B_V^T) / L, with w_s
// the window values (workgroup 0 only) and o'_s the weighted coordinates.
__global__ void __launch_bounds__(NT) k_decode_merge(const DecodeArgs a) {
  __shared__ float fac[MAXG][2];
  __shared__ float op[MAXG][D];  // merged o' (rsV <= D entries per head)
  __shared__ float ow[MAXG][D];  // merged window values
  const int ul = blockIdx.x, u = a.u0 + ul;
  const int g = a.L.g, rsV = a.L.X[1].r, tid = threadIdx.x;
  const int rs = 2 + rsV + D, ns = a.nsplit;
  const float *rec = a.spart + (size_t)ul * ns * g * rs;
  int li, bi, h;
  unit_coords(a, ul, li, bi, h);
  if (tid < g) {
    float M = -INFINITY;
    for (int s = 0; s < ns; s++) {
      const float *r = rec + ((size_t)s * g + tid) * rs;
      if (r[1] > 0.f) M = fmaxf(M, r[0]);
    }
    float L = 0.f;
    for (int s = 0; s < ns; s++) {
      const float *r = rec + ((size_t)s * g + tid) * rs;
      if (r[1] > 0.f) L += r[1] * ex2(r[0] - M);
    }
    fac[tid][0] = M;
    fac[tid][1] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < g * (rsV + D); idx += NT) {
    const int hh = idx / (rsV + D), t = idx - hh * (rsV + D);
    float v = 0.f;
    for (int s = 0; s < ns; s++) {
      const float *r = rec + ((size_t)s * g + hh) * rs;
      if (r[1] > 0.f) v += ex2(r[0] - fac[hh][0]) * r[2 + t];
    }
    if (t < rsV)
      op[hh][t] = v;
    else
      ow[hh][t - rsV] = v;
  }
  __syncthreads();
  const float *Bv = a.L.X[1].Bt + (size_t)u * rsV * D;
  float *out = (float *)a.out + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
  for (int idx = tid; idx < g * D; idx += NT) {
    const int hh = idx / D, t = idx - hh * D;
    float s = ow[hh][t];
    for (int j = 0; j < a.kV; j++) s += op[hh][j] * Bv[(size_t)j * D + t];
    out[idx] = s / fac[hh][1];
  }
}

template <int KS, int NTV, bool I8>
hipError_t launch_bf16_t(const DecodeArgs &a0, int nunits, hipStream_t s) {
  DecodeArgs a = a0;
  // stage the window in LDS when it fits next to the rest (160 KB per workgroup)
  const int ew = a.e + a.nnew;
  size_t lds = decode_unit_lds(a.L.X[0].r, a.L.X[1].r, a.L.g, ew);
  a.wlds = (ew > 0 && lds <= 160 * 1024 && ((uintptr_t)a.q & 15) == 0) ? 1 : 0;
  if (!a.wlds) lds = decode_unit_lds(a.L.X[0].r, a.L.X[1].r, a.L.g, 0);
  if (a.nsplit > 0) {
    hipError_t e = hipFuncSetAttribute((const void *)k_decode_unit<KS, NTV, true, I8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_decode_unit<KS, NTV, true, I8>), dim3(nunits, a.nsplit), dim3(NTU), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_decode_merge, dim3(nunits), dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  hipError_t e = hipFuncSetAttribute((const void *)k_decode_unit<KS, NTV, false, I8>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_unit<KS, NTV, false, I8>), dim3(nunits), dim3(NTU), lds, s, a);
  return hipGetLastError();
}

template <int KS, bool I8>
hipError_t launch_bf16_ks(const DecodeArgs &a, int nunits, hipStream_t s) {
  switch ((a.L.X[1].r + 15) / 16) {
    case 1: return launch_bf16_t<KS, 1, I8>(a, nunits, s);
    case 2: return launch_bf16_t<KS, 2, I8>(a, nunits, s);
    case 3: return launch_bf16_t<KS, 3, I8>(a, nunits, s);
    case 4: return launch_bf16_t<KS, 4, I8>(a, nunits, s);
    case 5: return launch_bf16_t<KS, 5, I8>(a, nunits, s);
    case 6: return launch_bf16_t<KS, 6, I8>(a, nunits, s);
    case 7: return launch_bf16_t<KS, 7, I8>(a, nunits, s);
    default: return launch_bf16_t<KS, 8, I8>(a, nunits, s);
  }
}

template <bool I8>
hipError_t launch_unit_path(const DecodeArgs &a, int nunits, hipStream_t s) {
  switch ((a.L.X[0].r + 31) / 32) {
    case 1: return launch_bf16_ks<1, I8>(a, nunits, s);
    case 2: return launch_bf16_ks<2, I8>(a, nunits, s);
    case 3: return launch_bf16_ks<3, I8>(a, nunits, s);
    default: return launch_bf16_ks<4, I8>(a, nunits, s);
  }
}

template <typename TC, typename TK>
hipError_t launch_decode_t(const DecodeArgs &a, int nunits, hipStream_t s) {
  const size_t lds = sizeof(float) * (4 * MAXG + QS_FLOATS + (size_t)MAXG * a.L.chunk);
  hipError_t e = hipFuncSetAttribute((const void *)k_decode<TC, TK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode<TC, TK>), dim3(a.nchunk + 1, nunits), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int decode_chunk_rows(const Layout &L) { return L.chunk; }

// the matrix-core decode: bf16 or int8 coordinates, bf16 rows, ranks in 8-column pieces
static bool unit_path(const Layout &L) {
  return (L.coord_bf16 || L.coord_i8) && L.kv_bf16 && L.X[0].r % 8 == 0 && L.X[1].r % 8 == 0;
}

bool decode_can_fuse(const DecodeArgs &a) {
  if (!unit_path(a.L)) return false;
  if ((((uintptr_t)a.q | (uintptr_t)a.nk | (uintptr_t)a.nv) & 15) != 0) return false;
  return decode_unit_lds(a.L.X[0].r, a.L.X[1].r, a.L.g, a.e + 1) <= 160 * 1024;
}

bool decode_can_split(const DecodeArgs &a) {
  if (!unit_path(a.L)) return false;
  return a.nnew == 0;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  const int nunits = a.L.batch * a.nl * a.L.kvh;
  if (unit_path(a.L)) return a.L.coord_i8 ? launch_unit_path<true>(a, nunits, s) : launch_unit_path<false>(a, nunits, s);
  if (a.L.coord_bf16 && a.L.kv_bf16) return launch_decode_t<uint16_t, uint16_t>(a, nunits, s);
  if (a.L.coord_bf16) return launch_decode_t<uint16_t, float>(a, nunits, s);
  if (a.L.kv_bf16) return launch_decode_t<float, uint16_t>(a, nunits, s);
  return launch_decode_t<float, float>(a, nunits, s);
}

}  // namespace iskv
