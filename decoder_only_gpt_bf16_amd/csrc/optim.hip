// Optimizer step: AdamW over a set of fp32 tensors with global-norm gradient
// clipping ("nanoGPT — Karpathy's minimal GPT pretraining repo", model.py
// section, configure_optimizers: weight decay on 2-D tensors only; train.py
// section: gradients clipped to a global norm before the step).  AdamW's
// update is the decoupled-weight-decay Adam of Loshchilov & Hutter
// ("Decoupled Weight Decay Regularization", Algorithm 2) with bias-corrected
// moments.
//
// Three kernels, all HBM-bound and deterministic:
//   sumsq_k   per 8192-element chunk, the sum of squared gradients (fp32 per
//             thread, fp64 across the block) into one partial per chunk;
//   norm_k    one block adds the partials in a fixed order, forms the norm
//             and the clip factor, and leaves both in the workspace;
//   adamw_k   per chunk, reads the factor and updates param, m, v (and the
//             optional bf16 copy of param) in one pass: 28 bytes per element
//             (30 with the bf16 copy).
// A launch covers up to OPT_TABLE tensors, whose descriptors travel in the
// kernel arguments; larger sets take several launches.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "kernels.h"

// Scratch of the allocation-free entry point (gpt_adamw_step_noalloc): the
// fp64 gradient-norm partial of each chunk, then the clip factor and the
// norm, laid out as launch_adamw lays out its workspace.  A file-scope
// device array: every GPU the library runs on holds its own copy until the
// process ends.  In host code the name is only a stand-in for the symbol;
// kernels get the device address that hipGetSymbolAddress returns for the
// current device (adamw_noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[ADAMW_NOALLOC_MAX_CHUNKS * sizeof(double) + 256];

namespace {

constexpr int OPT_THREADS = 256;
constexpr int OPT_CHUNK = 8192;  // elements per block: 8 float4 per thread

struct OptTable {
  float* p[OPT_TABLE];
  const float* g[OPT_TABLE];
  float* m[OPT_TABLE];
  float* v[OPT_TABLE];
  bf16* p16[OPT_TABLE];
  long n[OPT_TABLE];
  int decay[OPT_TABLE];
  int cstart[OPT_TABLE + 1];  // first chunk of each tensor within the launch
  int count;
};

__device__ __forceinline__ int table_slot(const OptTable& T, int blk) {
  int j = 0;
  while (j + 1 < T.count && blk >= T.cstart[j + 1]) ++j;
  return j;
}

// fixed-order tree sum of one double per thread over the block
__device__ double block_sum_d(double x) {
  __shared__ double red[OPT_THREADS];
  red[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int w = OPT_THREADS / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(OPT_THREADS) void sumsq_k(OptTable T, double* __restrict__ part) {
  const int j = table_slot(T, blockIdx.x);
  const long base = (long)(blockIdx.x - T.cstart[j]) * OPT_CHUNK;
  const long n = T.n[j];
  const float* g = T.g[j];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < OPT_CHUNK / (4 * OPT_THREADS); ++k) {
    const long e = base + 4L * (k * OPT_THREADS + threadIdx.x);
    if (e + 4 <= n) {
      const float4 x = *reinterpret_cast<const float4*>(g + e);
      s = fmaf(x.x, x.x, s); s = fmaf(x.y, x.y, s); s = fmaf(x.z, x.z, s); s = fmaf(x.w, x.w, s);
    } else {
      for (long i = e; i < n && i < e + 4; ++i) s = fmaf(g[i], g[i], s);
    }
  }
  const double t = block_sum_d((double)s);
  if (threadIdx.x == 0) part[blockIdx.x] = t;
}

// scal[0] = clip factor, scal[1] = global norm (before clipping).  Thread t
// adds partials t, t + 256, ... in index order; their loads are issued 32 at
// a time, since one block alone walks the whole partial array
__global__ __launch_bounds__(OPT_THREADS) void norm_k(const double* __restrict__ part, int nparts, float max_norm,
                                                      float* __restrict__ scal, float* __restrict__ norm_out) {
  constexpr int U = 32;
  double s = 0.0;
  int i = threadIdx.x;
  for (; i + (U - 1) * OPT_THREADS < nparts; i += U * OPT_THREADS) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = part[i + u * OPT_THREADS];
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  for (; i < nparts; i += OPT_THREADS) s += part[i];
  const double total = block_sum_d(s);
  if (threadIdx.x == 0) {
    const double norm = sqrt(total);
    const double f = (max_norm > 0.0f && norm > (double)max_norm) ? (double)max_norm / norm : 1.0;
    scal[0] = (float)f;
    scal[1] = (float)norm;
    if (norm_out) *norm_out = (float)norm;
  }
}

struct AdamHyper {
  float lr, b1, b2, eps, wd;
  float step_size;       // lr / (1 - b1^t)
  float inv_sqrt_bc2;    // 1 / sqrt(1 - b2^t)
};

__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v, const AdamHyper& h, float scale,
                                          bool decay) {
  g *= scale;
  m = fmaf(h.b1, m, (1.0f - h.b1) * g);
  v = fmaf(h.b2, v, (1.0f - h.b2) * g * g);
  const float denom = fmaf(sqrtf(v), h.inv_sqrt_bc2, h.eps);
  if (decay) p *= 1.0f - h.lr * h.wd;
  p -= h.step_size * (m / denom);
}

__global__ __launch_bounds__(OPT_THREADS) void adamw_k(OptTable T, const float* __restrict__ scal, AdamHyper h) {
  const int j = table_slot(T, blockIdx.x);
  const long base = (long)(blockIdx.x - T.cstart[j]) * OPT_CHUNK;
  const long n = T.n[j];
  float* p = T.p[j];
  const float* g = T.g[j];
  float* m = T.m[j];
  float* v = T.v[j];
  bf16* p16 = T.p16[j];
  const bool decay = T.decay[j] != 0;
  const float scale = scal ? scal[0] : 1.0f;
  // groups of G float4 per array: all loads of a group are issued before
  // any arithmetic, so 4 G vector loads are in flight per thread
  constexpr int G = 4, NK = OPT_CHUNK / (4 * OPT_THREADS);
#pragma unroll
  for (int k0 = 0; k0 < NK; k0 += G) {
    const long e0 = base + 4L * (k0 * OPT_THREADS + threadIdx.x);
    const long elast = e0 + 4L * (G - 1) * OPT_THREADS;
    if (elast + 4 <= n) {
      float4 pp[G], gg[G], mm[G], vv[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const long e = e0 + 4L * i * OPT_THREADS;
        pp[i] = *reinterpret_cast<const float4*>(p + e);
        gg[i] = *reinterpret_cast<const float4*>(g + e);
        mm[i] = *reinterpret_cast<const float4*>(m + e);
        vv[i] = *reinterpret_cast<const float4*>(v + e);
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const long e = e0 + 4L * i * OPT_THREADS;
        adam_elem(pp[i].x, gg[i].x, mm[i].x, vv[i].x, h, scale, decay);
        adam_elem(pp[i].y, gg[i].y, mm[i].y, vv[i].y, h, scale, decay);
        adam_elem(pp[i].z, gg[i].z, mm[i].z, vv[i].z, h, scale, decay);
        adam_elem(pp[i].w, gg[i].w, mm[i].w, vv[i].w, h, scale, decay);
        *reinterpret_cast<float4*>(p + e) = pp[i];
        *reinterpret_cast<float4*>(m + e) = mm[i];
        *reinterpret_cast<float4*>(v + e) = vv[i];
        if (p16) {
          bf16x4 b;
          b[0] = (bf16)pp[i].x; b[1] = (bf16)pp[i].y; b[2] = (bf16)pp[i].z; b[3] = (bf16)pp[i].w;
          *reinterpret_cast<bf16x4*>(p16 + e) = b;
        }
      }
    } else {
      for (int i = 0; i < G; ++i) {
        const long e = e0 + 4L * i * OPT_THREADS;
        for (long q = e; q < n && q < e + 4; ++q) {
          float pi = p[q], mi = m[q], vi = v[q];
          adam_elem(pi, g[q], mi, vi, h, scale, decay);
          p[q] = pi; m[q] = mi; v[q] = vi;
          if (p16) p16[q] = (bf16)pi;
        }
      }
    }
  }
}

long chunks_of(long n) { return (n + OPT_CHUNK - 1) / OPT_CHUNK; }

// tensors [first, last) into a launch table; returns its chunk count
int fill_table(const OptTensor* t, int first, int last, OptTable& T) {
  T = OptTable{};
  T.count = last - first;
  int c = 0;
  for (int i = first; i < last; ++i) {
    const int k = i - first;
    T.p[k] = t[i].p; T.g[k] = t[i].g; T.m[k] = t[i].m; T.v[k] = t[i].v;
    T.p16[k] = static_cast<bf16*>(t[i].p16);
    T.n[k] = t[i].n;
    T.decay[k] = t[i].decay;
    T.cstart[k] = c;
    c += (int)chunks_of(t[i].n);
  }
  for (int k = T.count; k <= OPT_TABLE; ++k) T.cstart[k] = c;
  return c;
}

}  // namespace

long adamw_chunks(const OptTensor* t, int count) {
  long c = 0;
  for (int i = 0; i < count; ++i) c += chunks_of(t[i].n);
  return c;
}

size_t adamw_ws_bytes(const OptTensor* t, int count) {
  return align256((size_t)adamw_chunks(t, count) * sizeof(double)) + 256;
}

hipError_t launch_adamw(const OptTensor* t, int count, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int step, float max_norm, float* norm_out, void* ws,
                        hipStream_t s) {
  const long total = adamw_chunks(t, count);
  double* part = static_cast<double*>(ws);
  float* scal = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)total * sizeof(double)));
  const bool need_norm = max_norm > 0.0f || norm_out;
  OptTable T;
  if (need_norm) {
    long done = 0;
    for (int first = 0; first < count; first += OPT_TABLE) {
      const int last = std::min(count, first + OPT_TABLE);
      const int c = fill_table(t, first, last, T);
      hipLaunchKernelGGL(sumsq_k, dim3(c), dim3(OPT_THREADS), 0, s, T, part + done);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      done += c;
    }
    hipLaunchKernelGGL(norm_k, dim3(1), dim3(OPT_THREADS), 0, s, part, (int)total, max_norm, scal, norm_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AdamHyper h;
  h.lr = lr; h.b1 = beta1; h.b2 = beta2; h.eps = eps; h.wd = weight_decay;
  h.step_size = (float)((double)lr / (1.0 - std::pow((double)beta1, (double)step)));
  h.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow((double)beta2, (double)step)));
  for (int first = 0; first < count; first += OPT_TABLE) {
    const int last = std::min(count, first + OPT_TABLE);
    const int c = fill_table(t, first, last, T);
    hipLaunchKernelGGL(adamw_k, dim3(c), dim3(OPT_THREADS), 0, s, T, max_norm > 0.0f ? scal : nullptr, h);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for the process.
hipError_t adamw_noalloc_scratch(void** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
