// Row norms (LayerNorm with gain/bias, parameter-free RMSNorm) forward and
// backward, and deterministic column sums (norm gain/bias and Linear bias
// gradients).  One wavefront per row: 16-byte coalesced loads, the row held
// in registers, butterfly-shuffle reductions.  HBM-bound.
#include "kernels.h"

namespace {

constexpr int ROWS_PER_BLOCK = 4;  // one row per wave, 4 waves per block
constexpr int MAX_VPL = 4;         // up to 64 * 8 * 4 = 2048 columns

// Eight storage elements of a row as loaded (one 16-byte vector for bf16,
// two for fp32), converted to fp32 only where used, so a wave keeps several
// rows' loads in flight in few registers.
template <typename T>
struct Raw8 {
  static constexpr int U = sizeof(T) / 2;
  uint4 u[U];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int i = 0; i < U; ++i) u[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < U; ++i) u[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ void get(float* f) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < U; ++i) {
        f[4 * i] = __uint_as_float(u[i].x); f[4 * i + 1] = __uint_as_float(u[i].y);
        f[4 * i + 2] = __uint_as_float(u[i].z); f[4 * i + 3] = __uint_as_float(u[i].w);
      }
    }
  }
};

// VPL = vectors of 8 columns per lane (C <= 512 VPL).
template <typename T, int KIND, bool ROPE, int VPL>
__global__ __launch_bounds__(256) void norm_fwd_k(int N, int C, const T* __restrict__ x,
                                                  const T* __restrict__ w, const T* __restrict__ b,
                                                  float eps, T* __restrict__ y, float* __restrict__ stats,
                                                  RopeJob rj) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const T* xr = x + (long)row * C;
  Raw8<T> v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (row < N && c < C) v[i].load(xr + c);
  }
  if constexpr (ROPE) {
    // the RoPE table while the row's loads are in flight
    const int n = rj.T * rj.half, nthr = gridDim.x * blockDim.x;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += nthr) rj.cs[e] = rope_entry(rj, e);
  }
  if (row >= N) return;
  float s = 0.0f;
  if constexpr (KIND == 0) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        float f[8];
        v[i].get(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += f[e];
      }
    }
  }
  const float mean = KIND == 0 ? wave_sum(s) / C : 0.0f;
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < C) {
      float f[8];
      v[i].get(f);
#pragma unroll
      for (int e = 0; e < 8; ++e) { float d = f[e] - mean; s2 += d * d; }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / C + eps);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = (lane + 64 * i) * 8;
    if (c < C) {
      float f[8], o[8];
      v[i].get(f);
      float wv[8], bv[8];
      if (KIND == 0) {
        if (w) Vec8<T>::load(w + c, wv); else for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
        if (b) Vec8<T>::load(b + c, bv); else for (int e = 0; e < 8; ++e) bv[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float h = (f[e] - mean) * rstd;
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
// (bias) per block into colpart[0][blk][C], colpart[1][blk][C].  A wave
// walks rows row, row + stride, ...; the next row's x, dy and resid loads
// are issued before the current row's reductions, so they are in flight
// while it computes and stores.
template <typename T, int KIND, bool COLS, int VPL>
__global__ __launch_bounds__(256) void norm_bwd_k(int N, int C, const T* __restrict__ x,
                                                  const T* __restrict__ w, const T* __restrict__ dy,
                                                  const T* __restrict__ resid, float eps,
                                                  T* __restrict__ dx, float* __restrict__ colpart) {
  constexpr bool want_cols = COLS;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * ROWS_PER_BLOCK;
  float cw[VPL][8], cb[VPL][8];
#pragma unroll
  for (int i = 0; i < VPL; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { cw[i][e] = 0.0f; cb[i][e] = 0.0f; }

  Raw8<T> nx[VPL], ng[VPL], nr[VPL];
  auto fetch = [&](int rw) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (rw < N && c < C) {
        nx[i].load(x + (long)rw * C + c);
        ng[i].load(dy + (long)rw * C + c);
        if (resid) nr[i].load(resid + (long)rw * C + c); else nr[i].zero();
      }
    }
  };
  int row = blockIdx.x * ROWS_PER_BLOCK + wave;
  fetch(row);
  for (; row < N; row += stride) {
    Raw8<T> rx[VPL], rg[VPL], rr[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) { rx[i] = nx[i]; rg[i] = ng[i]; rr[i] = nr[i]; }
    fetch(row + stride);
    float s = 0.0f;
    if constexpr (KIND == 0) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (c < C) {
          float f[8];
          rx[i].get(f);
#pragma unroll
          for (int e = 0; e < 8; ++e) s += f[e];
        }
      }
    }
    const float mean = KIND == 0 ? wave_sum(s) / C : 0.0f;
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        float f[8];
        rx[i].get(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) { float d = f[e] - mean; s2 += d * d; }
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(s2) / C + eps);
    float sg = 0.0f, sgx = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        float xv[8], g[8], wv[8];
        rx[i].get(xv);
        rg[i].get(g);
        if (KIND == 0 && w) Vec8<T>::load(w + c, wv); else for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float h = (xv[e] - mean) * rstd;
          if (want_cols) { cw[i][e] = fmaf(g[e], h, cw[i][e]); cb[i][e] += g[e]; }
          const float gw = g[e] * wv[e];
          sg += gw;
          sgx = fmaf(gw, h, sgx);
        }
      }
    }
    const float mg = KIND == 0 ? wave_sum(sg) / C : 0.0f;
    const float mgx = wave_sum(sgx) / C;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c < C) {
        float xv[8], g[8], wv[8], r[8], o[8];
        rx[i].get(xv);
        rg[i].get(g);
        rr[i].get(r);
        if (KIND == 0 && w) Vec8<T>::load(w + c, wv); else for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float h = (xv[e] - mean) * rstd;
          o[e] = fmaf(rstd, g[e] * wv[e] - mg - h * mgx, r[e]);
        }
        Vec8<T>::store(dx + (long)row * C + c, o);
      }
    }
  }
  if constexpr (!COLS) return;
  // reduce the 4 waves' column partials through LDS, fixed order
  __shared__ float red[ROWS_PER_BLOCK][2][64 * 8];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
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
// jobs of one launch: blocks [start[j], start[j + 1]) take job j
struct ColsumJobs {
  ColsumJob job[COLSUM_JOBS_MAX];
  int start[COLSUM_JOBS_MAX + 1];
  int n;
};
__global__ __launch_bounds__(CF_COLS * CF_SEGS) void colsum_finish_k(ColsumJobs J, int accumulate) {
  int j = 0;
  while (j + 1 < J.n && (int)blockIdx.x >= J.start[j + 1]) ++j;
  const int C = J.job[j].C, nblk = J.job[j].nblk;
  const float* __restrict__ part = J.job[j].part;
  float* __restrict__ out = J.job[j].out;
  const int lc = threadIdx.x % CF_COLS, seg = threadIdx.x / CF_COLS;
  const int c = (blockIdx.x - J.start[j]) * CF_COLS + lc;
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
                           const void* b, float eps, void* y, float* stats, hipStream_t s, const RopeJob* rope) {
  if (N <= 0) return hipSuccess;
  if (C <= 0 || C > 64 * 8 * MAX_VPL || C % 8) return hipErrorInvalidValue;
  dim3 grid(cdiv(N, ROWS_PER_BLOCK)), block(256);
  RopeJob rj{};
  const bool r = rope && rope->cs;
  if (r) rj = *rope;
  const int vpl = cdiv(C, 512);
#define NF(T, K, R, V) hipLaunchKernelGGL((norm_fwd_k<T, K, R, V>), grid, block, 0, s, N, C, (const T*)x, \
                                          (const T*)w, (const T*)b, eps, (T*)y, stats, rj)
#define NFV(T, K, R) do { switch (vpl) { case 1: NF(T, K, R, 1); break; case 2: NF(T, K, R, 2); break; \
                                         case 3: NF(T, K, R, 3); break; default: NF(T, K, R, 4); } } while (0)
#define NFR(T, K) do { if (r) NFV(T, K, true); else NFV(T, K, false); } while (0)
  if (dtype == 1) { if (kind == 0) NFR(bf16, 0); else NFR(bf16, 1); }
  else { if (kind == 0) NFR(float, 0); else NFR(float, 1); }
#undef NFR
#undef NFV
#undef NF
  return hipGetLastError();
}

hipError_t launch_norm_bwd(int dtype, int kind, int N, int C, const void* x, const void* w,
                           const void* dy, const void* resid, float eps, void* dx,
                           float* colpart, int want_cols, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (C <= 0 || C > 64 * 8 * MAX_VPL || C % 8) return hipErrorInvalidValue;
  dim3 grid(norm_bwd_blocks(N)), block(256);
  const int vpl = cdiv(C, 512);
#define NB(T, K, COLS, V) hipLaunchKernelGGL((norm_bwd_k<T, K, COLS, V>), grid, block, 0, s, N, C, (const T*)x, \
                                             (const T*)w, (const T*)dy, (const T*)resid, eps, (T*)dx, colpart)
#define NBV(T, K, COLS) do { switch (vpl) { case 1: NB(T, K, COLS, 1); break; case 2: NB(T, K, COLS, 2); break; \
                                            case 3: NB(T, K, COLS, 3); break; default: NB(T, K, COLS, 4); } } while (0)
  // column partials exist only for LayerNorm's gain and bias
  if (dtype == 1) {
    if (kind == 0) { if (want_cols) NBV(bf16, 0, true); else NBV(bf16, 0, false); }
    else NBV(bf16, 1, false);
  } else {
    if (kind == 0) { if (want_cols) NBV(float, 0, true); else NBV(float, 0, false); }
    else NBV(float, 1, false);
  }
#undef NBV
#undef NB
  return hipGetLastError();
}

hipError_t launch_colsum_finish_jobs(const ColsumJob* jobs, int n, int accumulate, hipStream_t s) {
  if (n < 0 || n > COLSUM_JOBS_MAX) return hipErrorInvalidValue;
  ColsumJobs J{};
  J.n = n;
  J.start[0] = 0;
  for (int j = 0; j < n; ++j) {
    J.job[j] = jobs[j];
    J.start[j + 1] = J.start[j] + cdiv(jobs[j].C, CF_COLS);
  }
  if (J.start[n] == 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_finish_k, dim3(J.start[n]), dim3(CF_COLS * CF_SEGS), 0, s, J, accumulate);
  return hipGetLastError();
}

hipError_t launch_colsum_finish(int C, int nblk, const float* part, float* out, int accumulate,
                                hipStream_t s) {
  const ColsumJob job{part, nblk, C, out};
  return launch_colsum_finish_jobs(&job, 1, accumulate, s);
}

size_t colsum_scratch_bytes(int N, int C) {
  return align256((size_t)cdiv(N, COLSUM_ROWS) * C * sizeof(float));
}

int colsum_part_blocks(int N) { return std::max(1, cdiv(N, COLSUM_ROWS)); }

hipError_t launch_colsum_part(int dtype, int N, int C, long ld, const void* x, float* part, hipStream_t s) {
  if (N <= 0 || C <= 0) return hipErrorInvalidValue;
  dim3 grid(cdiv(C, 256), colsum_part_blocks(N));
  if (dtype == 1)
    hipLaunchKernelGGL(colsum_part_k<bf16>, grid, dim3(256), 0, s, N, C, ld, (const bf16*)x, part, COLSUM_ROWS);
  else
    hipLaunchKernelGGL(colsum_part_k<float>, grid, dim3(256), 0, s, N, C, ld, (const float*)x, part, COLSUM_ROWS);
  return hipGetLastError();
}
