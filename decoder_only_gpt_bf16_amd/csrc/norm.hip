// Row norms (LayerNorm with gain/bias, parameter-free RMSNorm) forward and
// backward, and deterministic column sums (norm gain/bias and Linear bias
// gradients).  One wavefront per row: 16-byte coalesced loads, the row held
// in registers, butterfly-shuffle reductions.  HBM-bound.
#include "kernels.h"

namespace {

constexpr int ROWS_PER_BLOCK = 4;  // one row per wave, 4 waves per block
constexpr int MAX_VPL = 4;         // up to 64 * 8 * 4 = 2048 columns

template <typename T, int KIND>
__global__ __launch_bounds__(256) void norm_fwd_k(int N, int C, const T* __restrict__ x,
                                                  const T* __restrict__ w, const T* __restrict__ b,
                                                  float eps, T* __restrict__ y, float* __restrict__ stats) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const T* xr = x + (long)row * C;
  float v[MAX_VPL][8];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MAX_VPL; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < C) {
      Vec8<T>::load(xr + c, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    }
  }
  const float mean = KIND == 0 ? wave_sum(s) / C : 0.0f;
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < MAX_VPL; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < C) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { float d = v[i][e] - mean; s2 += d * d; }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / C + eps);
#pragma unroll
  for (int i = 0; i < MAX_VPL; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < C) {
      float o[8];
      float wv[8], bv[8];
      if (KIND == 0) {
        if (w) Vec8<T>::load(w + c, wv); else for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
        if (b) Vec8<T>::load(b + c, bv); else for (int e = 0; e < 8; ++e) bv[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float h = (v[i][e] - mean) * rstd;
        o[e] = KIND == 0 ? fmaf(h, wv[e], bv[e]) : h;
      }
      Vec8<T>::store(y + (long)row * C + c, o);
    }
  }
  if (stats && lane == 0) {
    stats[row] = mean;
    stats[N + row] = rstd;
  }
}

// dx = norm backward (+ resid); column partials of dy*xhat (gain) and dy
// (bias) per block into colpart[0][blk][C], colpart[1][blk][C].
template <typename T, int KIND, bool COLS>
__global__ __launch_bounds__(256) void norm_bwd_k(int N, int C, const T* __restrict__ x,
                                                  const T* __restrict__ w, const T* __restrict__ dy,
                                                  const T* __restrict__ resid, float eps,
                                                  T* __restrict__ dx, float* __restrict__ colpart) {
  constexpr bool want_cols = COLS;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float cw[MAX_VPL][8], cb[MAX_VPL][8];
#pragma unroll
  for (int i = 0; i < MAX_VPL; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { cw[i][e] = 0.0f; cb[i][e] = 0.0f; }

  for (int row = blockIdx.x * ROWS_PER_BLOCK + wave; row < N; row += gridDim.x * ROWS_PER_BLOCK) {
    const T* xr = x + (long)row * C;
    const T* gr = dy + (long)row * C;
    float xv[MAX_VPL][8], g[MAX_VPL][8];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < MAX_VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        Vec8<T>::load(xr + c, xv[i]);
        Vec8<T>::load(gr + c, g[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += xv[i][e];
      }
    }
    const float mean = KIND == 0 ? wave_sum(s) / C : 0.0f;
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < MAX_VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { float d = xv[i][e] - mean; s2 += d * d; }
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(s2) / C + eps);
    // xhat in xv; gw = dy * w in place of g after column partials
    float sg = 0.0f, sgx = 0.0f;
#pragma unroll
    for (int i = 0; i < MAX_VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        float wv[8];
        if (KIND == 0 && w) Vec8<T>::load(w + c, wv); else for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float h = (xv[i][e] - mean) * rstd;
          xv[i][e] = h;
          if (want_cols) { cw[i][e] = fmaf(g[i][e], h, cw[i][e]); cb[i][e] += g[i][e]; }
          const float gw = g[i][e] * wv[e];
          g[i][e] = gw;
          sg += gw;
          sgx = fmaf(gw, h, sgx);
        }
      }
    }
    const float mg = KIND == 0 ? wave_sum(sg) / C : 0.0f;
    const float mgx = wave_sum(sgx) / C;
#pragma unroll
    for (int i = 0; i < MAX_VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        float o[8], r[8];
        if (resid) Vec8<T>::load(resid + (long)row * C + c, r); else for (int e = 0; e < 8; ++e) r[e] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(rstd, g[i][e] - mg - xv[i][e] * mgx, r[e]);
        Vec8<T>::store(dx + (long)row * C + c, o);
      }
    }
  }
  if constexpr (!COLS) return;
  // reduce the 4 waves' column partials through LDS, fixed order
  __shared__ float red[ROWS_PER_BLOCK][2][64 * 8];
#pragma unroll
  for (int i = 0; i < MAX_VPL; ++i) {
    if (i > 0 && 64 * 8 * i >= C) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[wave][0][lane * 8 + e] = cw[i][e];
      red[wave][1][lane * 8 + e] = cb[i][e];
    }
    __syncthreads();
    for (int k = threadIdx.x; k < 2 * 512; k += 256) {
      const int which = k >> 9, idx = k & 511;
      const int col = 64 * 8 * i + idx;
      if (col < C) {
        float acc = 0.0f;
        for (int q = 0; q < ROWS_PER_BLOCK; ++q) acc += red[q][which][idx];
        colpart[((long)which * gridDim.x + blockIdx.x) * C + col] = acc;
      }
    }
    __syncthreads();
  }
}

// out[c] (+)= sum of part[b][c] over b < nblk.  A block takes CF_COLS
// columns; CF_SEGS threads per column each add a contiguous run of the
// partials in order, their loads issued CF_U at a time, and the runs' sums
// are then added in run order: a fixed order for any launch.
constexpr int CF_COLS = 16, CF_SEGS = 16, CF_U = 16;
__global__ __launch_bounds__(CF_COLS * CF_SEGS) void colsum_finish_k(int C, int nblk, const float* __restrict__ part,
                                                                     float* __restrict__ out, int accumulate) {
  const int lc = threadIdx.x % CF_COLS, seg = threadIdx.x / CF_COLS;
  const int c = blockIdx.x * CF_COLS + lc;
  const int per = (nblk + CF_SEGS - 1) / CF_SEGS;
  const int b1 = min(nblk, (seg + 1) * per);
  float s = 0.0f;
  if (c < C) {
    int b = seg * per;
    for (; b + CF_U <= b1; b += CF_U) {
      float v[CF_U];
#pragma unroll
      for (int u = 0; u < CF_U; ++u) v[u] = part[(long)(b + u) * C + c];
#pragma unroll
      for (int u = 0; u < CF_U; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += part[(long)b * C + c];
  }
  __shared__ float red[CF_SEGS][CF_COLS];
  red[seg][lc] = s;
  __syncthreads();
  if (seg == 0 && c < C) {
    float t = red[0][lc];
    for (int q = 1; q < CF_SEGS; ++q) t += red[q][lc];
    out[c] = accumulate ? out[c] + t : t;
  }
}

// Column sums of x [N, C] (ld) into per-block partials [nblk][C]; a thread
// adds its column over the block's rows in order, loads issued 16 at a time.
template <typename T>
__global__ __launch_bounds__(256) void colsum_part_k(int N, int C, long ld, const T* __restrict__ x,
                                                     float* __restrict__ part, int rows_per_blk) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int r0 = blockIdx.y * rows_per_blk;
  const int r1 = min(N, r0 + rows_per_blk);
  constexpr int U = 16;
  float s = 0.0f;
  int r = r0;
  for (; r + U <= r1; r += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = to_f32(x[(long)(r + u) * ld + c]);
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  for (; r < r1; ++r) s += to_f32(x[(long)r * ld + c]);
  part[(long)blockIdx.y * C + c] = s;
}

constexpr int COLSUM_ROWS = 64;

}  // namespace

int norm_bwd_blocks(int N) { return std::max(1, std::min(cdiv(N, ROWS_PER_BLOCK), 1024)); }

hipError_t launch_norm_fwd(int dtype, int kind, int N, int C, const void* x, const void* w,
                           const void* b, float eps, void* y, float* stats, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  dim3 grid(cdiv(N, ROWS_PER_BLOCK)), block(256);
#define NF(T, K) hipLaunchKernelGGL((norm_fwd_k<T, K>), grid, block, 0, s, N, C, (const T*)x, \
                                    (const T*)w, (const T*)b, eps, (T*)y, stats)
  if (dtype == 1) { if (kind == 0) NF(bf16, 0); else NF(bf16, 1); }
  else { if (kind == 0) NF(float, 0); else NF(float, 1); }
#undef NF
  return hipGetLastError();
}

hipError_t launch_norm_bwd(int dtype, int kind, int N, int C, const void* x, const void* w,
                           const void* dy, const void* resid, float eps, void* dx,
                           float* colpart, int want_cols, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  dim3 grid(norm_bwd_blocks(N)), block(256);
#define NB(T, K, COLS) hipLaunchKernelGGL((norm_bwd_k<T, K, COLS>), grid, block, 0, s, N, C, (const T*)x, \
                                          (const T*)w, (const T*)dy, (const T*)resid, eps, (T*)dx, colpart)
  // column partials exist only for LayerNorm's gain and bias
  if (dtype == 1) {
    if (kind == 0) { if (want_cols) NB(bf16, 0, true); else NB(bf16, 0, false); }
    else NB(bf16, 1, false);
  } else {
    if (kind == 0) { if (want_cols) NB(float, 0, true); else NB(float, 0, false); }
    else NB(float, 1, false);
  }
#undef NB
  return hipGetLastError();
}

hipError_t launch_colsum_finish(int C, int nblk, const float* part, float* out, int accumulate,
                                hipStream_t s) {
  hipLaunchKernelGGL(colsum_finish_k, dim3(cdiv(C, CF_COLS)), dim3(CF_COLS * CF_SEGS), 0, s, C, nblk, part, out,
                     accumulate);
  return hipGetLastError();
}

size_t colsum_scratch_bytes(int N, int C) {
  return align256((size_t)cdiv(N, COLSUM_ROWS) * C * sizeof(float));
}

hipError_t launch_colsum(int dtype, int N, int C, long ld, const void* x, float* out, int accumulate,
                         float* scratch, hipStream_t s) {
  if (N <= 0) {
    if (!accumulate) return hipMemsetAsync(out, 0, C * sizeof(float), s);
    return hipSuccess;
  }
  const int nblk = cdiv(N, COLSUM_ROWS);
  dim3 grid(cdiv(C, 256), nblk);
  if (dtype == 1)
    hipLaunchKernelGGL(colsum_part_k<bf16>, grid, dim3(256), 0, s, N, C, ld, (const bf16*)x, scratch, COLSUM_ROWS);
  else
    hipLaunchKernelGGL(colsum_part_k<float>, grid, dim3(256), 0, s, N, C, ld, (const float*)x, scratch, COLSUM_ROWS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_colsum_finish(C, nblk, scratch, out, accumulate, s);
}
