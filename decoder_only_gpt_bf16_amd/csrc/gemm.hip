// GEMM kernels: bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16) with LDS
// double buffering, and an fp32 SIMT kernel for fp32 storage.
//
// MFMA kernel layout
//   * 256 threads = 4 wavefronts arranged 2 (M) x 2 (N); block tile BM x BN,
//     k tile BK = 64; each wave owns (BM/2) x (BN/2) = TM x TN MFMA tiles.
//   * Both operands live in LDS as [row][64 k] bf16 (128-byte rows, eight
//     16-byte units); unit c of row r is stored at position c ^ (r & 7) so
//     that the 16-byte fragment reads of 8 consecutive rows hit distinct
//     banks.  An operand given k-major in HBM is transposed while it is
//     staged: each thread loads an 8 (k) x 8 (row) block with eight 16-byte
//     loads and writes eight 16-byte k-vectors.
//   * The MFMA is issued with the B tile as its first operand, so a lane's
//     16 accumulators hold one output row m (lane & 31) and 4 runs of 4
//     consecutive columns n: epilogues read bias/residual and write outputs
//     as 4-element vectors.
//   * Tiles are mapped so that blocks resident on one XCD (the hardware
//     deals block ids round-robin over 8 XCDs) work on neighbouring tiles
//     of a grouped order and share their operand rows in that XCD's L2.
#include <type_traits>
#include "kernels.h"

namespace {

constexpr int BK = 64;
constexpr int NTHREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- epilogues
template <typename T>
__device__ __forceinline__ void load4(const T* p, float* f) {
  if constexpr (sizeof(T) == 2) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* f) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v;
    v[0] = (bf16)f[0]; v[1] = (bf16)f[1]; v[2] = (bf16)f[2]; v[3] = (bf16)f[3];
    *reinterpret_cast<bf16x4*>(p) = v;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
}

// Elementwise epilogue for 4 consecutive columns n..n+3 of row m.
template <typename T, int EPI>
__device__ __forceinline__ void epi4(const GemmParams& p, int m, int n, float* v) {
  if (m >= p.M || n >= p.N) return;
  const bool full = (n + 4 <= p.N);
  float t[4];
  if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
    if (p.bias) {
      const T* b = reinterpret_cast<const T*>(p.bias) + n;
      if (full) { load4<T>(b, t); for (int e = 0; e < 4; ++e) v[e] += t[e]; }
      else for (int e = 0; e < 4; ++e) if (n + e < p.N) v[e] += to_f32(b[e]);
    }
  }
  if constexpr (EPI == EPI_STORE) {
    if (p.resid) {
      const T* r = reinterpret_cast<const T*>(p.resid) + (long)m * p.ldr + n;
      if (full) { load4<T>(r, t); for (int e = 0; e < 4; ++e) v[e] += t[e]; }
      else for (int e = 0; e < 4; ++e) if (n + e < p.N) v[e] += to_f32(r[e]);
    }
    T* o = reinterpret_cast<T*>(p.out) + (long)m * p.ldc + n;
    if (full) store4<T>(o, v);
    else for (int e = 0; e < 4; ++e) if (n + e < p.N) o[e] = from_f32<T>(v[e]);
  } else if constexpr (EPI == EPI_GELU) {
    float g[4];
    for (int e = 0; e < 4; ++e) g[e] = gelu_f(v[e]);
    T* o = reinterpret_cast<T*>(p.out) + (long)m * p.ldc + n;
    T* o2 = reinterpret_cast<T*>(p.out2) + (long)m * p.ldc + n;
    if (full) { store4<T>(o, v); store4<T>(o2, g); }
    else for (int e = 0; e < 4; ++e) if (n + e < p.N) { o[e] = from_f32<T>(v[e]); o2[e] = from_f32<T>(g[e]); }
  } else if constexpr (EPI == EPI_GELU_BWD) {
    const T* u = reinterpret_cast<const T*>(p.aux) + (long)m * p.ldaux + n;
    T* o = reinterpret_cast<T*>(p.out) + (long)m * p.ldc + n;
    if (full) {
      load4<T>(u, t);
      for (int e = 0; e < 4; ++e) v[e] *= gelu_grad_f(t[e]);
      store4<T>(o, v);
    } else {
      for (int e = 0; e < 4; ++e) if (n + e < p.N) o[e] = from_f32<T>(v[e] * gelu_grad_f(to_f32(u[e])));
    }
  } else if constexpr (EPI == EPI_F32) {
    float* o = reinterpret_cast<float*>(p.out) + (long)blockIdx.z * p.split_stride + (long)m * p.ldc + n;
    if (full && (p.ldc & 3) == 0) {
      if (p.accumulate) { load4<float>(o, t); for (int e = 0; e < 4; ++e) v[e] += t[e]; }
      store4<float>(o, v);
    } else {
      for (int e = 0; e < 4; ++e) if (n + e < p.N) o[e] = p.accumulate ? o[e] + v[e] : v[e];
    }
  } else if constexpr (EPI == EPI_XENT_GRAD) {
    const float l = p.lse[m];
    const int tg = p.tgt[m] - p.col_offset;
    for (int e = 0; e < 4; ++e) {
      float pr = exp2f((v[e] - l) * LOG2E);
      v[e] = (pr - (n + e == tg ? 1.0f : 0.0f)) * p.scale;
    }
    T* o = reinterpret_cast<T*>(p.out) + (long)m * p.ldc + n;
    if (full) store4<T>(o, v);
    else for (int e = 0; e < 4; ++e) if (n + e < p.N) o[e] = from_f32<T>(v[e]);
  }
}

// Block id -> (tile_m, tile_n): XCD-aware remap, then grouped ordering.
__device__ __forceinline__ void tile_coords(const GemmParams& p, int& tm, int& tn) {
  const int nb = gridDim.x;
  int b = blockIdx.x;
  {
    const int xcd = b & 7, idx = b >> 3;
    const int per = nb >> 3, rem = nb & 7;
    b = xcd * per + min(xcd, rem) + idx;
  }
  constexpr int GROUP_M = 8;
  const int width = GROUP_M * p.tiles_n;
  const int group = b / width;
  const int first_m = group * GROUP_M;
  const int gsize = min(p.tiles_m - first_m, GROUP_M);
  const int r = b - group * width;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// ------------------------------------------------------------ staging
// Operand with k contiguous in HBM: R rows x 64 k, thread t covers unit
// c = t & 7 of rows (t >> 3) + 32 i.
template <int R>
struct StageKc {
  static constexpr int NV = R / 32;
  uint4 v[NV];
  __device__ __forceinline__ void load(const bf16* X, long ld, int r0, int rmax, int k0, int kend) {
    const int t = threadIdx.x;
    const int c = t & 7;
    const int kk = k0 + 8 * c;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int gr = r0 + (t >> 3) + 32 * i;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (gr < rmax) {
        const bf16* src = X + (long)gr * ld + kk;
        if (kk + 8 <= kend) {
          u = *reinterpret_cast<const uint4*>(src);
        } else if (kk < kend) {
          uint16_t h[8];
          for (int e = 0; e < 8; ++e)
            h[e] = (kk + e < kend) ? reinterpret_cast<const uint16_t*>(src)[e] : (uint16_t)0;
          u = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16), h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
        }
      }
      v[i] = u;
    }
  }
  __device__ __forceinline__ void store(uint4* lds) const {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int row = (t >> 3) + 32 * i;
      lds[row * 8 + (c ^ (row & 7))] = v[i];
    }
  }
};

// Operand with rows contiguous in HBM ([K][ld]): 8 x 8 sub-blocks
// s = t + 256 i, kg = s & 7 (k rows 8kg..8kg+7), rg = s >> 3 (rows 8rg..).
template <int R>
struct StageKm {
  static constexpr int NS = (R + 255) / 256;
  uint4 v[NS][8];
  __device__ __forceinline__ void load(const bf16* X, long ld, int r0, int rmax, int k0, int kend) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = t + 256 * i;
      const int kg = s & 7, rg = s >> 3;
      const int gr = r0 + 8 * rg;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + 8 * kg + j;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (s < R && gk < kend && gr < rmax) {
          const bf16* src = X + (long)gk * ld + gr;
          if (gr + 8 <= rmax) {
            u = *reinterpret_cast<const uint4*>(src);
          } else {
            uint16_t h[8];
            for (int e = 0; e < 8; ++e)
              h[e] = (gr + e < rmax) ? reinterpret_cast<const uint16_t*>(src)[e] : (uint16_t)0;
            u = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16), h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
          }
        }
        v[i][j] = u;
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = t + 256 * i;
      if (s >= R) continue;
      const int kg = s & 7, rg = s >> 3;
      const uint32_t* w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = reinterpret_cast<const uint32_t*>(&v[i][j]);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        // element rr of each k-row j, packed in k order
        const int word = rr >> 1;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t lo = w[2 * q][word], hi = w[2 * q + 1][word];
          o[q] = (rr & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int row = 8 * rg + rr;
        lds[row * 8 + (kg ^ rr)] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

template <bool KMAJ, int R>
using Stage = typename std::conditional<KMAJ, StageKm<R>, StageKc<R>>::type;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

// ------------------------------------------------------------ MFMA kernel
template <bool A_KMAJ, bool B_KMAJ, int EPI, int BM, int BN>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_mfma(GemmParams p) {
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int STAGE_UNITS = (BM + BN) * 8;
  __shared__ uint4 lds[2 * STAGE_UNITS];

  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * p.k_split;
  const int kend = min(p.K, kbeg + p.k_split);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = (wave & 1) * (BM / 2);
  const int wn = (wave >> 1) * (BN / 2);

  const bf16* A = reinterpret_cast<const bf16*>(p.A);
  const bf16* B = reinterpret_cast<const bf16*>(p.B);

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  Stage<A_KMAJ, BM> sa;
  Stage<B_KMAJ, BN> sb;
  if (nk > 0) {
    sa.load(A, p.lda, m0, p.M, kbeg, kend);
    sb.load(B, p.ldb, n0, p.N, kbeg, kend);
    sa.store(lds);
    sb.store(lds + BM * 8);
  }
  __syncthreads();

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kbeg + (kt + 1) * BK;
      sa.load(A, p.lda, m0, p.M, k0, kend);
      sb.load(B, p.ldb, n0, p.N, k0, kend);
    }
    const uint4* As = lds + cur * STAGE_UNITS;
    const uint4* Bs = As + BM * 8;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int unit = (2 * kk + lhalf) ^ (lrow & 7);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(As[(wm + 32 * i + lrow) * 8 + unit]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = as_bf16x8(Bs[(wn + 32 * j + lrow) * 8 + unit]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[j][i], 0, 0, 0);
    }
    if (more) {
      uint4* nxt = lds + (cur ^ 1) * STAGE_UNITS;
      sa.store(nxt);
      sb.store(nxt + BM * 8);
    }
    __syncthreads();
  }

  // lane holds row m = m0 + wm + 32 i + lrow and columns
  // n = n0 + wn + 32 j + 8 g + 4 lhalf + e (register 4 g + e).
  if constexpr (EPI == EPI_XENT_STATS) {
    const int nbase = n0 + wn;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm + 32 * i + lrow;
      const int tg = (m < p.M) ? p.tgt[m] - p.col_offset : -1;
      float mx = -INFINITY, zt = 0.0f;
      bool have = false;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = nbase + 32 * j + 8 * (r >> 2) + 4 * lhalf + (r & 3);
          const float v = acc[j][i][r];
          if (n < p.N) mx = fmaxf(mx, v);
          if (n == tg) { zt = v; have = true; }
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float s = 0.0f;
      if (mx != -INFINITY) {
        const float ms = mx * LOG2E;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int n = nbase + 32 * j + 8 * (r >> 2) + 4 * lhalf + (r & 3);
            if (n < p.N) s += exp2f(fmaf(acc[j][i][r], LOG2E, -ms));
          }
      }
      s += __shfl_xor(s, 32, 64);
      if (m < p.M) {
        if (have) p.ztgt[m] = zt;
        if (lhalf == 0) p.part[(long)m * p.part_ld + p.part_off + nbase / (BN / 2)] = make_float2(mx, s);
      }
    }
  } else {
    using OutT = bf16;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm + 32 * i + lrow;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn + 32 * j + 8 * g + 4 * lhalf;
          float v[4] = {acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]};
          epi4<OutT, EPI>(p, m, n, v);
        }
      }
  }
}

// ------------------------------------------------------------ SIMT kernel
// 64 x 64 tile, k tile 16, 256 threads each computing 4 x 4 outputs in fp32.
template <typename T, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(256) void gemm_simt(GemmParams p) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int ty = t >> 4, tx = t & 15;
  const int kbeg = blockIdx.z * p.k_split;
  const int kend = min(p.K, kbeg + p.k_split);
  const T* A = reinterpret_cast<const T*>(p.A);
  const T* B = reinterpret_cast<const T*>(p.B);
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = t + 256 * q;
      int r, k;
      if (A_KMAJ) { k = e >> 6; r = e & 63; } else { r = e >> 4; k = e & 15; }
      const int gm = m0 + r, gk = k0 + k;
      float va = 0.0f;
      if (gm < p.M && gk < kend) va = to_f32(A_KMAJ ? A[(long)gk * p.lda + gm] : A[(long)gm * p.lda + gk]);
      As[k][r] = va;
      if (B_KMAJ) { k = e >> 6; r = e & 63; } else { r = e >> 4; k = e & 15; }
      const int gn = n0 + r;
      const int gk2 = k0 + k;
      float vb = 0.0f;
      if (gn < p.N && gk2 < kend) vb = to_f32(B_KMAJ ? B[(long)gk2 * p.ldb + gn] : B[(long)gn * p.ldb + gk2]);
      Bs[k][r] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[k][ty * 4 + i]; b[i] = Bs[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    epi4<T, EPI>(p, m0 + ty * 4 + i, n0 + tx * 4, v);
  }
}

// Sum of split-K partials [S][M][N] into out (fp32, ldc), fixed order.
__global__ void splitk_reduce(const float* part, int S, long stride, int M, int N, float* out,
                              long ldc, int accumulate) {
  const long total = (long)M * N;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int z = 0; z < S; ++z) s += part[z * stride + e];
    const long m = e / N, n = e - m * N;
    float* o = out + m * ldc + n;
    *o = accumulate ? *o + s : s;
  }
}

struct Plan {
  int BMv, BNv, splits, k_split;
};

// Tile size and split-K choice for the MFMA path.
Plan plan_mfma(const GemmDesc& d) {
  Plan pl;
  const long t256 = (long)cdiv(d.M, 256) * cdiv(d.N, 256);
  if (d.epi == EPI_XENT_STATS || t256 >= 240) { pl.BMv = 256; pl.BNv = 256; }
  else { pl.BMv = 128; pl.BNv = 128; }
  const long tiles = (long)cdiv(d.M, pl.BMv) * cdiv(d.N, pl.BNv);
  pl.splits = 1;
  if (d.epi == EPI_F32) {
    // weight gradients: small output, long K -> split K to fill 256 CUs
    while (tiles * pl.splits < 200 && d.K / (pl.splits * 2) >= 512) pl.splits *= 2;
  }
  pl.k_split = cdiv(cdiv(d.K, pl.splits), BK) * BK;
  pl.splits = cdiv(d.K, pl.k_split);
  return pl;
}

template <bool AK, bool BKm, int EPI, int BMv, int BNv>
hipError_t go_mfma(const GemmParams& p, int splits, hipStream_t s) {
  dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
  hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, BMv, BNv>), grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

template <bool AK, bool BKm, int EPI>
hipError_t go_mfma_tiles(const GemmParams& p, const Plan& pl, hipStream_t s) {
  if (pl.BMv == 256) return go_mfma<AK, BKm, EPI, 256, 256>(p, pl.splits, s);
  return go_mfma<AK, BKm, EPI, 128, 128>(p, pl.splits, s);
}

template <typename T, bool AK, bool BKm, int EPI>
hipError_t go_simt(const GemmParams& p, int splits, hipStream_t s) {
  dim3 grid(cdiv(p.N, 64), cdiv(p.M, 64), splits);
  hipLaunchKernelGGL((gemm_simt<T, AK, BKm, EPI>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

GemmParams make_params(const GemmDesc& d) {
  GemmParams p{};
  p.A = d.A; p.B = d.B; p.lda = d.lda; p.ldb = d.ldb;
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.out = d.out; p.ldc = d.ldc; p.split_stride = 0;
  p.bias = d.bias; p.resid = d.resid; p.ldr = d.ldr; p.out2 = d.out2;
  p.aux = d.aux; p.ldaux = d.ldaux; p.accumulate = d.accumulate;
  p.tgt = d.tgt; p.col_offset = d.col_offset; p.part = d.part; p.part_ld = d.part_ld;
  p.part_off = d.part_off; p.ztgt = d.ztgt; p.lse = d.lse; p.scale = d.scale;
  return p;
}

}  // namespace

int xent_part_cols() { return 128; }

size_t gemm_split_scratch_bytes(const GemmDesc& d, int dtype) {
  if (dtype != 1 || d.epi != EPI_F32) return 0;
  Plan pl = plan_mfma(d);
  if (pl.splits <= 1) return 0;
  return align256((size_t)pl.splits * d.M * d.N * sizeof(float));
}

hipError_t launch_gemm(const GemmDesc& d, int dtype, void* ws, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  GemmParams p = make_params(d);
  if (dtype == 1) {
    Plan pl = plan_mfma(d);
    p.tiles_m = cdiv(d.M, pl.BMv);
    p.tiles_n = cdiv(d.N, pl.BNv);
    p.k_split = pl.k_split;
    if (d.K <= 0) { pl.splits = 1; p.k_split = 0; }
    const bool split = pl.splits > 1;
    if (split) {
      p.out = ws; p.ldc = d.N; p.accumulate = 0; p.split_stride = (long)d.M * d.N;
    }
    hipError_t e = hipErrorInvalidValue;
    const bool ak = d.a_kmaj, bk = d.b_kmaj;
    switch (d.epi) {
      case EPI_STORE:
        if (!ak && !bk) e = go_mfma_tiles<false, false, EPI_STORE>(p, pl, s);
        else if (!ak && bk) e = go_mfma_tiles<false, true, EPI_STORE>(p, pl, s);
        break;
      case EPI_GELU:
        if (!ak && !bk) e = go_mfma_tiles<false, false, EPI_GELU>(p, pl, s);
        break;
      case EPI_GELU_BWD:
        if (!ak && bk) e = go_mfma_tiles<false, true, EPI_GELU_BWD>(p, pl, s);
        break;
      case EPI_F32:
        if (ak && bk) e = go_mfma_tiles<true, true, EPI_F32>(p, pl, s);
        else if (!ak && bk) e = go_mfma_tiles<false, true, EPI_F32>(p, pl, s);
        else if (!ak && !bk) e = go_mfma_tiles<false, false, EPI_F32>(p, pl, s);
        break;
      case EPI_XENT_STATS:
        if (!ak && !bk) e = go_mfma<false, false, EPI_XENT_STATS, 256, 256>(p, pl.splits, s);
        break;
      case EPI_XENT_GRAD:
        if (!ak && !bk) e = go_mfma_tiles<false, false, EPI_XENT_GRAD>(p, pl, s);
        break;
    }
    if (e != hipSuccess) return e;
    if (split) {
      const long total = (long)d.M * d.N;
      int blocks = (int)std::min<long>((total + 255) / 256, 4096);
      hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, s, (const float*)ws, pl.splits,
                         (long)d.M * d.N, d.M, d.N, (float*)d.out, d.ldc, d.accumulate);
      e = hipGetLastError();
    }
    return e;
  }
  // fp32 storage: SIMT kernel, no split.
  p.k_split = d.K > 0 ? d.K : 0;
  const bool ak = d.a_kmaj, bk = d.b_kmaj;
  switch (d.epi) {
    case EPI_STORE:
      if (!ak && !bk) return go_simt<float, false, false, EPI_STORE>(p, 1, s);
      if (!ak && bk) return go_simt<float, false, true, EPI_STORE>(p, 1, s);
      break;
    case EPI_GELU:
      if (!ak && !bk) return go_simt<float, false, false, EPI_GELU>(p, 1, s);
      break;
    case EPI_GELU_BWD:
      if (!ak && bk) return go_simt<float, false, true, EPI_GELU_BWD>(p, 1, s);
      break;
    case EPI_F32:
      if (ak && bk) return go_simt<float, true, true, EPI_F32>(p, 1, s);
      if (!ak && bk) return go_simt<float, false, true, EPI_F32>(p, 1, s);
      if (!ak && !bk) return go_simt<float, false, false, EPI_F32>(p, 1, s);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}
