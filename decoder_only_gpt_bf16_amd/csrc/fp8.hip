// FP8 quantization and GEMM on the gfx950 8-bit MFMA ("Train your own
// ChatGPT", 6.2, FP8 paragraph; the nanochat-d20 card's Pretraining row:
// matmuls in 8-bit floats with a dynamic per-tensor scale).  OCP formats:
// E4M3 (largest 448) and E5M2 (largest 57344).
//
// Quantization (HBM-bound, two passes): amax_k takes max |x| per 4096-element
// chunk, amax_finish_k forms amax, scale = fmt_max / amax (1 when amax = 0)
// and 1 / scale; quant_k writes the codes of clamp(x * scale) rounded to
// nearest even by v_cvt_pk_{fp8,bf8}_f32.
//
// GEMM: C[m][n] = sum_k A[m][k] B[n][k] / (scale_a scale_b), both operands
// k-contiguous bytes, bf16 output.  256 x 256 tiles, 8 waves of 128 x 64,
// k tile 128 bytes staged global -> LDS by direct copies into 128-byte rows of
// eight 16-byte units (XOR-swizzled as in the bf16 GEMM), two stages.  One
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) per 64 k: a lane
// brings 32 bytes of its row; A and B fragments take the same four of the
// row's units (which of the 64 k a byte stands for only has to agree between
// the operands, since the instruction pairs byte j of lane (row, half) of one
// operand with byte j of the same half of the other).
#include "kernels.h"

namespace {

struct Q2dJobs {
  const bf16* x[Q2D_MAX];
  uint8_t* q[Q2D_MAX];
  uint8_t* qT[Q2D_MAX];
  long ldT[Q2D_MAX];
  int R[Q2D_MAX], Cc[Q2D_MAX], tiles_c[Q2D_MAX];
  int start[Q2D_MAX + 1];
  float* scal[Q2D_MAX];
  int n;
};

constexpr int Q_THREADS = 256;
constexpr int Q_CHUNK = 4096;  // elements per block: 16 per thread

__device__ __forceinline__ float fp8_max(int fmt) { return fmt == FP8_E5M2 ? 57344.0f : 448.0f; }

__global__ __launch_bounds__(Q_THREADS) void amax_k(long n, const bf16* __restrict__ x, float* __restrict__ part) {
  const long base = (long)blockIdx.x * Q_CHUNK + 8L * threadIdx.x;
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const long e = base + (long)k * 8 * Q_THREADS;
    float v[8];
    if (e + 8 <= n) {
      Vec8<bf16>::load(x + e, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    } else {
      for (long i = e; i < n && i < e + 8; ++i) m = fmaxf(m, fabsf(to_f32(x[i])));
    }
  }
  m = wave_max(m);
  __shared__ float red[Q_THREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int w = 1; w < Q_THREADS / 64; ++w) t = fmaxf(t, red[w]);
    part[blockIdx.x] = t;
  }
}

// scal[0] = scale, scal[1] = amax, scal[2] = 1 / scale
__global__ __launch_bounds__(Q_THREADS) void amax_finish_k(int nparts, const float* __restrict__ part, int fmt,
                                                           float* __restrict__ scal) {
  // one block walks all partials: their loads go out 16 at a time
  constexpr int U = 16;
  float m = 0.0f;
  int i = threadIdx.x;
  for (; i + (U - 1) * Q_THREADS < nparts; i += U * Q_THREADS) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = part[i + u * Q_THREADS];
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, v[u]);
  }
  for (; i < nparts; i += Q_THREADS) m = fmaxf(m, part[i]);
  m = wave_max(m);
  __shared__ float red[Q_THREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float amax = red[0];
    for (int w = 1; w < Q_THREADS / 64; ++w) amax = fmaxf(amax, red[w]);
    const float scale = amax > 0.0f ? fp8_max(fmt) / amax : 1.0f;
    scal[0] = scale;
    scal[1] = amax;
    scal[2] = 1.0f / scale;
  }
}

template <int FMT, bool HI>
__device__ __forceinline__ int cvt_pair(float a, float b, int old) {
  if constexpr (FMT == FP8_E5M2) return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
  else return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

template <int FMT>
__global__ __launch_bounds__(Q_THREADS) void quant_k(long n, const bf16* __restrict__ x, const float* __restrict__ scal,
                                                     uint8_t* __restrict__ q) {
  const float s = scal[0];
  const float mx = FMT == FP8_E5M2 ? 57344.0f : 448.0f;
  const long base = (long)blockIdx.x * Q_CHUNK + 8L * threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const long e = base + (long)k * 8 * Q_THREADS;
    if (e + 8 <= n) {
      float v[8];
      Vec8<bf16>::load(x + e, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i] * s, -mx), mx);
      int lo = cvt_pair<FMT, false>(v[0], v[1], 0);
      lo = cvt_pair<FMT, true>(v[2], v[3], lo);
      int hi = cvt_pair<FMT, false>(v[4], v[5], 0);
      hi = cvt_pair<FMT, true>(v[6], v[7], hi);
      *reinterpret_cast<uint2*>(q + e) = make_uint2((uint32_t)lo, (uint32_t)hi);
    } else {
      for (long i = e; i < n && i < e + 8; ++i) {
        const float v = fminf(fmaxf(to_f32(x[i]) * s, -mx), mx);
        q[i] = (uint8_t)(cvt_pair<FMT, false>(v, 0.0f, 0) & 0xff);
      }
    }
  }
}

// Codes of up to Q2D_MAX bf16 matrices x_j [R_j][Cc_j] (Cc_j a multiple of
// 16), one per-tensor scale each, of one format.  Two launches:
//   amax_parts_k: AMAX_PARTS blocks per matrix, each the max |x| over a
//     grid-stride share of its 8-element vectors (8 loads in flight);
//   quant2d_k: 64 x 64 tiles; every block first reduces its matrix's
//     AMAX_PARTS partials (4 KB) into amax and scale = fmt_max / amax (1 when
//     amax is 0), the first block of a matrix also stores (scale, amax,
//     1 / scale); then q [R][Cc] codes (when given) by 8-byte row stores and
//     the transpose qT [Cc][ldT] (when given) through a 4 KB LDS tile by
//     16-byte row stores, qT columns R .. ldT - 1 zero.
constexpr int AMAX_PARTS = 1024;

__global__ __launch_bounds__(256) void amax_parts_k(Q2dJobs J, float* __restrict__ part) {
  const int j = blockIdx.x / AMAX_PARTS, b = blockIdx.x % AMAX_PARTS;
  const long nv = (long)J.R[j] * J.Cc[j] / 8;
  const bf16* x = J.x[j];
  float m = 0.0f;
  constexpr long STRIDE = 256L * AMAX_PARTS;
  for (long v0 = (long)b * 256 + threadIdx.x; v0 < nv; v0 += 8 * STRIDE) {
    uint4 f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long v = v0 + u * STRIDE;
      f[u] = v < nv ? *reinterpret_cast<const uint4*>(x + 8 * v) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t w4[4] = {f[u].x, f[u].y, f[u].z, f[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w4[e] << 16)), fabsf(__uint_as_float(w4[e] & 0xffff0000u))));
    }
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int FMT>
__global__ __launch_bounds__(256) void quant2d_k(Q2dJobs J, const float* __restrict__ part) {
  __shared__ uint32_t tile[64][17];  // 64 rows x 64 codes, padded row
  __shared__ float red[4];
  int j = 0;
#pragma unroll
  for (int i = 1; i < Q2D_MAX; ++i)
    if (i < J.n && (int)blockIdx.x >= J.start[i]) j = i;
  const int tid = blockIdx.x - J.start[j];
  const int R = J.R[j], Cc = J.Cc[j];
  const int r0 = (tid / J.tiles_c[j]) * 64, c0 = (tid % J.tiles_c[j]) * 64;
  const int t = threadIdx.x;
  // amax and scale of matrix j from its partials (same value in every block)
  const float* pj = part + (long)j * AMAX_PARTS;
  float m = fmaxf(fmaxf(pj[t], pj[t + 256]), fmaxf(pj[t + 512], pj[t + 768]));
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float mx = FMT == FP8_E5M2 ? 57344.0f : 448.0f;
  const float s = amax > 0.0f ? mx / amax : 1.0f;
  if (tid == 0 && t == 0) {
    J.scal[j][0] = s;
    J.scal[j][1] = amax;
    J.scal[j][2] = 1.0f / s;
  }
  uint8_t* q = J.q[j];
  uint8_t* qT = J.qT[j];
  const bf16* x = J.x[j];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int rr = t / 8 + 32 * v, cc = 8 * (t % 8);
    const int r = r0 + rr, c = c0 + cc;
    uint32_t lo = 0, hi = 0;
    if (r < R && c < Cc) {
      float f[8];
      Vec8<bf16>::load(x + (long)r * Cc + c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(f[i] * s, -mx), mx);
      int a = cvt_pair<FMT, false>(f[0], f[1], 0);
      a = cvt_pair<FMT, true>(f[2], f[3], a);
      int b = cvt_pair<FMT, false>(f[4], f[5], 0);
      b = cvt_pair<FMT, true>(f[6], f[7], b);
      lo = (uint32_t)a;
      hi = (uint32_t)b;
      if (q) *reinterpret_cast<uint2*>(q + (long)r * Cc + c) = make_uint2(lo, hi);
    }
    tile[rr][cc / 4] = lo;
    tile[rr][cc / 4 + 1] = hi;
  }
  if (!qT) return;
  __syncthreads();
  // output row c0 + jj of qT: bytes r0 + 16 g .. + 15 (source rows) of
  // source column jj; thread t: jj = t / 4, g = t % 4
  const int jj = t / 4, g = t % 4;
  const long ldT = J.ldT[j];
  if (c0 + jj >= Cc || r0 + 16 * g >= ldT) return;
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t code = (tile[16 * g + 4 * k + e][jj / 4] >> (8 * (jj % 4))) & 0xffu;
      word |= code << (8 * e);
    }
    w[k] = word;
  }
  *reinterpret_cast<uint4*>(qT + (long)(c0 + jj) * ldT + r0 + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------ GEMM
constexpr int F_BM = 256, F_BN = 256, F_NT = 512, F_BK = 128;  // BK in bytes (elements)
constexpr int F_TM = 4, F_TN = 2;                              // 32 x 32 tiles per wave (128 x 64)
constexpr uint32_t F_OOB = 0x80000000u;

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int fswz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

struct Fp8GemmParams {
  const uint8_t* A;
  const uint8_t* B;
  long lda, ldb, ldc;
  int M, N, K;
  uint32_t a_bytes, b_bytes;
  bf16* out;
  const float* scal_a;
  const float* scal_b;
  int tiles_n;
};

// 256 rows x 128 bytes of a k-contiguous operand into LDS [row][8 units]:
// instruction i of wave w fills physical units P = (8 i + w) * 64 + lane,
// row P / 8, slot P % 8 holding logical unit (P % 8) ^ fswz(row)
__device__ __forceinline__ void f_stage(uint4* lds, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int rmax, int k0,
                                        int K) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < F_BM * 8 / F_NT; ++i) {
    const int P = (8 * i + w) * 64 + lane;
    const int row = P >> 3;
    const int u = (P & 7) ^ fswz(row);
    const int gr = r0 + row, kk = k0 + 16 * u;
    const uint32_t off = (kk + 16 <= K && gr < rmax) ? (uint32_t)((long)gr * ld + kk) : F_OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + (8 * i + w) * 64),
                                             16, off, 0, 0, 0);
  }
}

// 32 bytes of tile row `row` for k-step ks (0, 1) and lane half hf: units
// 4 ks + hf and 4 ks + 2 + hf
__device__ __forceinline__ v8i f_frag(const uint4* lds, int row, int ks, int hf) {
  const uint4 a = lds[row * 8 + ((4 * ks + hf) ^ fswz(row))];
  const uint4 b = lds[row * 8 + ((4 * ks + 2 + hf) ^ fswz(row))];
  v8i v;
  v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  return v;
}

template <int FA, int FB>
__global__ __launch_bounds__(F_NT, 1) void gemm_fp8_k(Fp8GemmParams p) {
  __shared__ uint4 lds[2 * (F_BM + F_BN) * 8];
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
  const int m0 = tm * F_BM, n0 = tn * F_BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;
  const int lrow = lane & 31, hf = lane >> 5;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), (short)0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.B), (short)0, (int)p.b_bytes, 0x00020000);
  f32x16 acc[F_TN][F_TM];
#pragma unroll
  for (int j = 0; j < F_TN; ++j)
#pragma unroll
    for (int i = 0; i < F_TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;
  const int nk = (p.K + F_BK - 1) / F_BK;
  auto issue = [&](int t) {
    uint4* st = lds + (t & 1) * (F_BM + F_BN) * 8;
    f_stage(st, ra, p.lda, m0, p.M, t * F_BK, p.K);
    f_stage(st + F_BM * 8, rb, p.ldb, n0, p.N, t * F_BK, p.K);
  };
  issue(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) issue(t + 1);
    const uint4* As = lds + (t & 1) * (F_BM + F_BN) * 8;
    const uint4* Bs = As + F_BM * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i a[F_TM], b[F_TN];
#pragma unroll
      for (int i = 0; i < F_TM; ++i) a[i] = f_frag(As, wm + 32 * i + lrow, ks, hf);
#pragma unroll
      for (int j = 0; j < F_TN; ++j) b[j] = f_frag(Bs, wn + 32 * j + lrow, ks, hf);
#pragma unroll
      for (int j = 0; j < F_TN; ++j)
#pragma unroll
        for (int i = 0; i < F_TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[j][i], FB, FA, 0, 127, 0, 127);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  // lane: output row m = lrow of each 32-row strip, columns 8 g + 4 hf + e
  const float inv = p.scal_a[2] * p.scal_b[2];
#pragma unroll
  for (int i = 0; i < F_TM; ++i) {
    const int m = m0 + wm + 32 * i + lrow;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < F_TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn + 32 * j + 8 * g + 4 * hf;
        if (n >= p.N) continue;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[j][i][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(p.out + (long)m * p.ldc + n) = o;
      }
  }
}

}  // namespace

long fp8_amax_parts(long n) { return (n + Q_CHUNK - 1) / Q_CHUNK; }

hipError_t launch_fp8_quantize(long n, const void* x, int fmt, void* q, float* scal, float* part, hipStream_t s) {
  const long nb = fp8_amax_parts(n);
  hipLaunchKernelGGL(amax_k, dim3((unsigned)nb), dim3(Q_THREADS), 0, s, n, (const bf16*)x, part);
  hipLaunchKernelGGL(amax_finish_k, dim3(1), dim3(Q_THREADS), 0, s, (int)nb, (const float*)part, fmt, scal);
  if (fmt == FP8_E5M2)
    hipLaunchKernelGGL(quant_k<FP8_E5M2>, dim3((unsigned)nb), dim3(Q_THREADS), 0, s, n, (const bf16*)x,
                       (const float*)scal, (uint8_t*)q);
  else
    hipLaunchKernelGGL(quant_k<FP8_E4M3>, dim3((unsigned)nb), dim3(Q_THREADS), 0, s, n, (const bf16*)x,
                       (const float*)scal, (uint8_t*)q);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(int M, int N, int K, const void* A, long lda, int fa, const float* scal_a, const void* B,
                           long ldb, int fb, const float* scal_b, void* out, long ldc, hipStream_t s) {
  Fp8GemmParams p{};
  p.A = static_cast<const uint8_t*>(A); p.B = static_cast<const uint8_t*>(B);
  p.lda = lda; p.ldb = ldb; p.ldc = ldc; p.M = M; p.N = N; p.K = K;
  p.a_bytes = (uint32_t)((long)(M - 1) * lda + K);
  p.b_bytes = (uint32_t)((long)(N - 1) * ldb + K);
  p.out = static_cast<bf16*>(out); p.scal_a = scal_a; p.scal_b = scal_b;
  p.tiles_n = cdiv(N, F_BN);
  dim3 grid(cdiv(M, F_BM) * p.tiles_n);
#define FG(a, b) hipLaunchKernelGGL((gemm_fp8_k<a, b>), grid, dim3(F_NT), 0, s, p)
  if (fa == FP8_E4M3 && fb == FP8_E4M3) FG(FP8_E4M3, FP8_E4M3);
  else if (fa == FP8_E5M2 && fb == FP8_E4M3) FG(FP8_E5M2, FP8_E4M3);
  else if (fa == FP8_E4M3 && fb == FP8_E5M2) FG(FP8_E4M3, FP8_E5M2);
  else FG(FP8_E5M2, FP8_E5M2);
#undef FG
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_2d(const Fp8Q2d* d, int n, int fmt, float* part, hipStream_t s) {
  if (n <= 0 || n > Q2D_MAX) return hipErrorInvalidValue;
  Q2dJobs J{};
  J.n = n;
  int tiles = 0;
  for (int i = 0; i < n; ++i) {
    const Fp8Q2d& e = d[i];
    if (e.R <= 0 || e.Cc <= 0 || e.Cc % 16 || (e.qT && (e.ldT < e.R || e.ldT % 64))) return hipErrorInvalidValue;
    J.x[i] = static_cast<const bf16*>(e.x);
    J.q[i] = static_cast<uint8_t*>(e.q);
    J.qT[i] = static_cast<uint8_t*>(e.qT);
    J.ldT[i] = e.ldT;
    J.R[i] = e.R;
    J.Cc[i] = e.Cc;
    J.scal[i] = e.scal;
    J.tiles_c[i] = cdiv(e.Cc, 64);
    J.start[i] = tiles;
    // with the transpose, the tiles cover the padded rows R .. ldT - 1 too (zeros)
    tiles += J.tiles_c[i] * cdiv(e.qT ? e.ldT : (long)e.R, 64);
  }
  for (int i = n; i <= Q2D_MAX; ++i) J.start[i] = tiles;
  hipLaunchKernelGGL(amax_parts_k, dim3(n * AMAX_PARTS), dim3(256), 0, s, J, part);
  if (fmt == FP8_E5M2)
    hipLaunchKernelGGL(quant2d_k<FP8_E5M2>, dim3(tiles), dim3(256), 0, s, J, (const float*)part);
  else
    hipLaunchKernelGGL(quant2d_k<FP8_E4M3>, dim3(tiles), dim3(256), 0, s, J, (const float*)part);
  return hipGetLastError();
}
