// Cross-entropy reductions and the bits-per-byte reduction.
//
// Cross-entropy ("nanoGPT — Karpathy's minimal GPT pretraining repo",
// train.py: mean over tokens of the negative log-probability of the next
// token): per token, nats = logsumexp(z) - z[target].  The bf16 path gets
// (max, sum exp) partials per 64-column block from the LM-head GEMM
// epilogue; xent_finish_k merges them per row.  The fp32 path materialises
// one vocabulary chunk of logits at a time and keeps running statistics.
//
// Bits per byte ("Train your own ChatGPT", 6.2, loss_eval.py paragraph):
// sum of nats over tokens whose target has a non-zero byte length, divided by
// ln 2 times the sum of those byte lengths; zero-length (special) tokens are
// excluded from both sums.  A single workgroup reduces in a fixed order.
#include "kernels.h"

namespace {

constexpr int FINISH_ROWS = 4;  // rows (waves) per block

__device__ __forceinline__ void merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}

// One wave per row: lse from the row's P (max, sum exp) partials, nats =
// lse - z[target] (NaN when the target lies outside [0, V): no tile wrote its
// logit).  Per-block sum of the (weighted) nats into loss_part[block] (waves
// in fixed order).  A lane takes partials lane, lane + 64, ... in batches of
// XB with all of a batch's loads issued before any arithmetic, and folds
// each batch into its (max, sum) with one exponential per partial.
constexpr int XB = 16;

__global__ __launch_bounds__(256) void xent_finish_k(int N, int P, int V, const float2* __restrict__ part,
                                                     const int32_t* __restrict__ tgt,
                                                     const float* __restrict__ ztgt, const float* __restrict__ w,
                                                     float* __restrict__ lse, float* __restrict__ nats,
                                                     float* __restrict__ loss_part) {
  __shared__ float red[FINISH_ROWS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * FINISH_ROWS + wave;
  float nat = 0.0f;
  if (row < N) {
    const float2* pr = part + (long)row * P;
    float m = -INFINITY, s = 0.0f;
    for (int p0 = 0; p0 < P; p0 += 64 * XB) {
      float2 v[XB];
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int p = p0 + lane + 64 * i;
        v[i] = p < P ? pr[p] : make_float2(-INFINITY, 0.0f);
      }
      float mb = m;
#pragma unroll
      for (int i = 0; i < XB; ++i) mb = fmaxf(mb, v[i].x);
      if (mb != -INFINITY) {
        float sb = s * expf(m - mb);
#pragma unroll
        for (int i = 0; i < XB; ++i) sb = fmaf(v[i].y, expf(v[i].x - mb), sb);
        m = mb;
        s = sb;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
      merge(m, s, m2, s2);
    }
    const float l = m + logf(s);
    const int t = tgt[row];
    nat = (t >= 0 && t < V) ? l - ztgt[row] : __builtin_nanf("");
    if (lane == 0) {
      lse[row] = l;
      nats[row] = nat;
    }
  }
  float term = nat;
  if (w && row < N) term = w[row] != 0.0f ? w[row] * nat : 0.0f;
  if (lane == 0) red[wave] = (row < N) ? term : 0.0f;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int w = 0; w < FINISH_ROWS; ++w) t += red[w];
    loss_part[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(1024) void loss_sum_k(int nblk, const float* __restrict__ part, float scale,
                                                   float* __restrict__ loss) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 1024) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(red[0] * scale);
}

// Generic path: update running (max, sum exp) of each row with one fp32
// logit chunk z[:, 0:Vc] (global columns v0..v0+Vc), pick the target logit.
__global__ __launch_bounds__(256) void xent_rows_stats_k(int N, int Vc, int v0, const float* __restrict__ z,
                                                         long ldz, const int32_t* __restrict__ tgt,
                                                         float2* __restrict__ run, float* __restrict__ ztgt,
                                                         int first) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const float* zr = z + (long)row * ldz;
  float m = -INFINITY;
  for (int c = lane; c < Vc; c += 64) m = fmaxf(m, zr[c]);
  m = wave_max(m);
  float s = 0.0f;
  for (int c = lane; c < Vc; c += 64) s += expf(zr[c] - m);
  s = wave_sum(s);
  if (lane == 0) {
    if (!first) {
      const float2 r = run[row];
      merge(m, s, r.x, r.y);
    }
    run[row] = make_float2(m, s);
    const int t = tgt[row] - v0;
    if (t >= 0 && t < Vc) ztgt[row] = zr[t];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void xent_rows_grad_k(int N, int Vc, int v0, const float* __restrict__ z, long ldz,
                                                        const int32_t* __restrict__ tgt, const float* __restrict__ lse,
                                                        float scale, const float* __restrict__ w, T* __restrict__ dz,
                                                        long lddz) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)N * Vc) return;
  const int row = (int)(idx / Vc), c = (int)(idx % Vc);
  const float p = expf(z[(long)row * ldz + c] - lse[row]);
  const float g = (p - (c + v0 == tgt[row] ? 1.0f : 0.0f)) * (w ? scale * w[row] : scale);
  dz[(long)row * lddz + c] = from_f32<T>(g);
}

template <typename T>
__global__ void f32_to_k(long n, const float* __restrict__ src, T* __restrict__ dst) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = from_f32<T>(src[i]);
}

__global__ __launch_bounds__(1024) void bpb_k(int N, int V, const float* __restrict__ nats, const int32_t* __restrict__ tg,
                                              const int32_t* __restrict__ tb, double* __restrict__ sum_nats,
                                              int64_t* __restrict__ sum_bytes) {
  __shared__ double rn[1024];
  __shared__ long long rb[1024];
  double sn = 0.0;
  long long sb = 0;
  for (int i = threadIdx.x; i < N; i += 1024) {
    const int t = tg[i];
    const int nb = (t >= 0 && t < V) ? tb[t] : 0;
    if (nb > 0) {
      sn += (double)nats[i];
      sb += nb;
    }
  }
  rn[threadIdx.x] = sn;
  rb[threadIdx.x] = sb;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      rn[threadIdx.x] += rn[threadIdx.x + w];
      rb[threadIdx.x] += rb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *sum_nats += rn[0];
    *sum_bytes += (int64_t)rb[0];
  }
}

}  // namespace

int xent_finish_blocks(int N) { return cdiv(N, FINISH_ROWS); }

hipError_t launch_xent_finish(int N, int P, int V, const float2* part, const int32_t* tgt, const float* ztgt,
                              const float* w, float* lse, float* nats, float* loss_part, hipStream_t s) {
  hipLaunchKernelGGL(xent_finish_k, dim3(xent_finish_blocks(N)), dim3(256), 0, s, N, P, V, part, tgt, ztgt, w, lse,
                     nats, loss_part);
  return hipGetLastError();
}

hipError_t launch_loss_sum(int nblk, const float* loss_part, float scale, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_sum_k, dim3(1), dim3(1024), 0, s, nblk, loss_part, scale, loss);
  return hipGetLastError();
}

hipError_t launch_xent_rows_stats(int N, int Vc, int v0, const float* z, long ldz, const int32_t* tgt, float2* run,
                                  float* ztgt, int first, hipStream_t s) {
  hipLaunchKernelGGL(xent_rows_stats_k, dim3(cdiv(N, 4)), dim3(256), 0, s, N, Vc, v0, z, ldz, tgt, run, ztgt, first);
  return hipGetLastError();
}

hipError_t launch_xent_rows_grad(int dtype, int N, int Vc, int v0, const float* z, long ldz, const int32_t* tgt,
                                 const float* lse, float scale, const float* w, void* dz, long lddz, hipStream_t s) {
  dim3 grid((unsigned)cdiv((long)N * Vc, 256));
  if (dtype == 1)
    hipLaunchKernelGGL(xent_rows_grad_k<bf16>, grid, dim3(256), 0, s, N, Vc, v0, z, ldz, tgt, lse, scale, w, (bf16*)dz,
                       lddz);
  else
    hipLaunchKernelGGL(xent_rows_grad_k<float>, grid, dim3(256), 0, s, N, Vc, v0, z, ldz, tgt, lse, scale, w, (float*)dz,
                       lddz);
  return hipGetLastError();
}

hipError_t launch_f32_to(int dtype, long n, const float* src, void* dst, hipStream_t s) {
  dim3 grid((unsigned)std::min<long>(cdiv(n, 256), 8192));
  if (dtype == 1) hipLaunchKernelGGL(f32_to_k<bf16>, grid, dim3(256), 0, s, n, src, (bf16*)dst);
  else hipLaunchKernelGGL(f32_to_k<float>, grid, dim3(256), 0, s, n, src, (float*)dst);
  return hipGetLastError();
}

hipError_t launch_bpb(int N, int V, const float* nats, const int32_t* targets, const int32_t* token_bytes,
                      double* sum_nats, int64_t* sum_bytes, hipStream_t s) {
  hipLaunchKernelGGL(bpb_k, dim3(1), dim3(1024), 0, s, N, V, nats, targets, token_bytes, sum_nats, sum_bytes);
  return hipGetLastError();
}
