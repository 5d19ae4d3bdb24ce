// GEMM kernels: bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16) with LDS
// double buffering, and an fp32 SIMT kernel for fp32 storage.
//
// MFMA kernel layout
//   * Block tile BM x BN, k tile BK = 64, two LDS stages.  256 x 256 tiles
//     run 8 wavefronts (2 along M x 4 along N, two per SIMD); 128 x 128
//     tiles run 4 (2 x 2).  A wave owns TM x TN MFMA tiles of 32 x 32.
//   * Operand tiles go global -> LDS with buffer loads that write LDS
//     directly (no staging registers); rows and k beyond the matrix read as
//     zeros through the buffer's range check, so the copies carry no
//     branches.  k-contiguous operands are stored [row][64 k] (128-byte
//     rows), k-major operands as they lie in HBM ([64 k][rows]) and are read
//     transposed with ds_read_b64_tr_b16.  16-byte units are XOR-swizzled
//     per row so that both read patterns are free of bank conflicts.
//   * The MFMA is issued with the B tile as its first operand, so a lane's
//     16 accumulators hold one output row m (lane & 31) and 4 runs of 4
//     consecutive columns n.  The epilogue stages each 32-row strip through
//     LDS and applies bias / residual / GELU / GELU' / cross-entropy
//     arithmetic on 8-column row vectors.
//   * Tiles are mapped so that blocks resident on one XCD (the hardware
//     deals block ids round-robin over 8 XCDs) work on neighbouring tiles
//     of a grouped order and share their operand rows in that XCD's L2.
#include <type_traits>
#include "kernels.h"

namespace {

constexpr int BK = 64;
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

template <typename T, int W>
__device__ __forceinline__ void loadW(const T* p, float* f) {
  if constexpr (W == 8) {
    Vec8<T>::load(p, f);
  } else {
    load4<T>(p, f);
  }
}
template <typename T, int W>
__device__ __forceinline__ void storeW(T* p, const float* f) {
  if constexpr (W == 8) {
    Vec8<T>::store(p, f);
  } else {
    store4<T>(p, f);
  }
}

// Elementwise epilogue for W consecutive columns n..n+W-1 of row m.  Partial
// vectors (n + W > N) take the same arithmetic with guarded element access.
template <typename T, int EPI, int W>
__device__ __forceinline__ void epiW(const GemmParams& p, int m, int n, float* v, bool use_pre = false,
                                     uint4 pre = uint4{}) {
  if (m >= p.M || n >= p.N) return;
  const bool full = (n + W <= p.N);
  float t[W];
  // use_pre: pre holds the row vector of resid (EPI_STORE) or aux
  // (EPI_GELU_BWD) at (m, n), loaded ahead by the caller (bf16, W == 8, full
  // vectors only)
  auto take_pre = [&](float* f) {
    const uint32_t w4[4] = {pre.x, pre.y, pre.z, pre.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w4[i] << 16);
      f[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
    }
  };
  if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
    if (p.bias) {
      const T* b = reinterpret_cast<const T*>(p.bias) + n;
      if (full) loadW<T, W>(b, t);
      else for (int e = 0; e < W; ++e) t[e] = (n + e < p.N) ? to_f32(b[e]) : 0.0f;
      for (int e = 0; e < W; ++e) v[e] += t[e];
    }
  }
  if constexpr (EPI == EPI_STORE) {
    if (p.resid) {
      const T* r = reinterpret_cast<const T*>(p.resid) + (long)m * p.ldr + n;
      if (full && use_pre) take_pre(t);
      else if (full) loadW<T, W>(r, t);
      else for (int e = 0; e < W; ++e) t[e] = (n + e < p.N) ? to_f32(r[e]) : 0.0f;
      for (int e = 0; e < W; ++e) v[e] += t[e];
    }
  } else if constexpr (EPI == EPI_GELU) {
    // out2 = GELU(u) feeds the next GEMM; out = GELU'(u) is what the
    // backward needs of u, so it is stored in u's place
    float g[W];
    for (int e = 0; e < W; ++e) gelu_and_grad(v[e], g[e], v[e]);
    T* o2 = reinterpret_cast<T*>(p.out2) + (long)m * p.ldc + n;
    if (full) storeW<T, W>(o2, g);
    else for (int e = 0; e < W; ++e) if (n + e < p.N) o2[e] = from_f32<T>(g[e]);
    if (!p.out) return;  // forward only: nothing keeps GELU'(u)
  } else if constexpr (EPI == EPI_GELU_BWD) {
    const T* dg = reinterpret_cast<const T*>(p.aux) + (long)m * p.ldaux + n;
    if (full && use_pre) take_pre(t);
    else if (full) loadW<T, W>(dg, t);
    else for (int e = 0; e < W; ++e) t[e] = (n + e < p.N) ? to_f32(dg[e]) : 0.0f;
    for (int e = 0; e < W; ++e) v[e] *= t[e];
  } else if constexpr (EPI == EPI_XENT_GRAD) {
    const float l = p.lse[m];
    const int tg = p.tgt[m] - p.col_offset;
    const float sc = p.roww ? p.scale * p.roww[m] : p.scale;
    for (int e = 0; e < W; ++e) {
      const float pr = exp2f((v[e] - l) * LOG2E);
      v[e] = (pr - (n + e == tg ? 1.0f : 0.0f)) * sc;
    }
  }
  if constexpr (EPI == EPI_F32) {
    float* o = reinterpret_cast<float*>(p.out) + (long)blockIdx.z * p.split_stride + (long)m * p.ldc + n;
    if (full && (p.ldc & 3) == 0) {
      if (p.accumulate) { loadW<float, W>(o, t); for (int e = 0; e < W; ++e) v[e] += t[e]; }
      storeW<float, W>(o, v);
    } else {
      for (int e = 0; e < W; ++e) if (n + e < p.N) o[e] = p.accumulate ? o[e] + v[e] : v[e];
    }
  } else {
    T* o = reinterpret_cast<T*>(p.out) + (long)m * p.ldc + n;
    if constexpr (EPI == EPI_GELU && W == 8 && sizeof(T) == 2) {
      // GELU'(u) is read only by the backward: a non-temporal store keeps
      // its 8 N C bytes from crowding the next GEMM's operands out of the
      // caches (that GEMM, proj, measured 7 us faster this way)
      if (full) {
        bf16x8 q;
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (bf16)v[e];
        __builtin_nontemporal_store(q, reinterpret_cast<bf16x8*>(o));
      } else {
        for (int e = 0; e < W; ++e) if (n + e < p.N) o[e] = from_f32<T>(v[e]);
      }
    } else {
      if (full) storeW<T, W>(o, v);
      else for (int e = 0; e < W; ++e) if (n + e < p.N) o[e] = from_f32<T>(v[e]);
    }
  }
}

// Block id -> (tile_m, tile_n): XCD-aware remap, then grouped ordering.
__device__ __forceinline__ void tile_coords(const GemmParams& p, int bid, int nb, int& tm, int& tn) {
  int b = bid;
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
// Operands are read with raw buffer loads: a lane whose 16-byte vector lies
// outside the matrix (row >= rows, k >= kend) gets an offset beyond the
// buffer's record count and the hardware returns zeros, so the loads carry
// no branches and stay in flight together.  Extents along the contiguous
// dimension are multiples of 8 elements (checked on the host).
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS swizzles (16-byte units, XOR by row) chosen so that the fragment
// reads below are free of bank conflicts on a 64-bank LDS:
//   k-contiguous tiles, 128-byte rows: f(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
//   k-major tiles, 256/512-byte rows:   f(r) = ((r & 3) << 2) | ((r >> 2) & 3)
__device__ __forceinline__ int swz128(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swzq(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
//   k-major tiles, 320-byte rows (20 units): f(r) = (r >> 2) & 3 (stays in range)
//   k-major tiles, 384-byte rows (24 units): f(r) = ((r >> 1) & 1) << 2 (below 8,
//     so it stays in range; the row stride is 32 banks mod 64, and within
//     each aligned group of four k-rows the two even and the two odd rows
//     take opposite halves of their 32 banks)
//   k-major tiles, 640-byte rows (40 units): f(r) = tab[r & 15] < 8, found by
//   search over such tables
template <int UPR>
__device__ __forceinline__ int swz_km(int r) {
  if constexpr (UPR == 20) {
    return (r >> 2) & 3;
  } else if constexpr (UPR == 24) {
    return ((r >> 1) & 1) << 2;
  } else if constexpr (UPR == 40) {
    constexpr uint64_t tab = 0x6433054362356005ull;  // nibble i = f(i): 5,0,0,6,5,3,2,6,3,4,5,0,3,3,4,6
    return (int)((tab >> (4 * (r & 15))) & 0xf);
  } else {
    return swzq(r);
  }
}

// Asynchronous global -> LDS copy of 16 bytes per lane: lane L's vector
// lands at LDS byte address lds_base + 16 L (lds_base wave-uniform); an
// out-of-range offset writes zeros.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Operand with k contiguous in HBM: R rows x 64 k, LDS [row][8 units].
// Direct copy by NT threads: wave w's instruction i fills physical units
// P = ((NT / 64) i + w) * 64 + lane, i.e. row P / 8, slot P % 8, which holds
// logical unit (P % 8) ^ f(row).
template <int R, int NT>
struct StageKc {
  // copy instructions per thread; when R * 8 units are not a multiple of the
  // thread count, the last one is issued by the first waves only
  static constexpr int NL = (R * 8 + NT - 1) / NT;
  // copy instruction i alone
  static __device__ __forceinline__ void direct1(uint4* lds, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int rmax,
                                                 int k0, int kend, int i) {
    static_assert(R % 8 == 0, "tile rows a multiple of 8");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if ((R * 8) % NT != 0 && NT / 64 * i + w >= R * 8 / 64) return;
    const int P = (NT / 64 * i + w) * 64 + lane;
    const int row = P >> 3;
    const int u = (P & 7) ^ swz128(row);
    const int gr = r0 + row, kk = k0 + 8 * u;
    const uint32_t off = (kk + 8 <= kend && gr < rmax) ? (uint32_t)(((long)gr * ld + kk) * 2) : OOB;
    load_lds16(rs, lds + (NT / 64 * i + w) * 64, off);
  }
  static __device__ __forceinline__ void direct(uint4* lds, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int rmax,
                                                int k0, int kend) {
#pragma unroll
    for (int i = 0; i < NL; ++i) direct1(lds, rs, ld, r0, rmax, k0, kend, i);
  }
  // A/B operand fragment: tile row `row`, k-step kk, lane half hf
  static __device__ __forceinline__ bf16x8 frag(const uint4* lds, int row, int kk, int lane) {
    return __builtin_bit_cast(bf16x8, lds[row * 8 + ((2 * kk + (lane >> 5)) ^ swz128(row))]);
  }
};

// Operand with rows contiguous in HBM ([K][ld]): staged as-is, LDS
// [64 k][R / 8 units], and read transposed with ds_read_b64_tr_b16: within a
// 16-lane group, lane i receives element i % 4 of the 4-element vectors
// addressed by lanes 4 q + i / 4 (q = 0..3).  Direct copy: physical unit P is
// k-row P / UPR, slot P % UPR, holding logical unit (P % UPR) ^ f(k-row).
template <int R, int NT>
struct StageKm {
  static constexpr int UPR = R / 8;
  static constexpr int NL = (64 * UPR + NT - 1) / NT;  // as in StageKc
  static __device__ __forceinline__ void direct1(uint4* lds, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int rmax,
                                                 int k0, int kend, int i) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if ((64 * UPR) % NT != 0 && NT / 64 * i + w >= UPR) return;
    const int P = (NT / 64 * i + w) * 64 + lane;
    const int kr = P / UPR;
    const int c = (P % UPR) ^ swz_km<UPR>(kr);
    const int gk = k0 + kr, gc = r0 + 8 * c;
    const uint32_t off = (gk < kend && gc + 8 <= rmax) ? (uint32_t)(((long)gk * ld + gc) * 2) : OOB;
    load_lds16(rs, lds + (NT / 64 * i + w) * 64, off);
  }
  static __device__ __forceinline__ void direct(uint4* lds, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int rmax,
                                                int k0, int kend) {
#pragma unroll
    for (int i = 0; i < NL; ++i) direct1(lds, rs, ld, r0, rmax, k0, kend, i);
  }
  static __device__ __forceinline__ i16x4 tr(const uint4* lds, int krow, int col) {
    const bf16* base = reinterpret_cast<const bf16*>(lds);
    const int off = (krow * UPR + ((col >> 3) ^ swz_km<UPR>(krow))) * 8 + (col & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(base + off));
  }
  // fragment of tile column `row` (an m or n index): k slots 16 kk + 8 hf + 0..7
  // (the swizzles have period 16 in the k-row, so k-step kk only adds a
  // constant offset of 16 rows)
  static __device__ __forceinline__ bf16x8 frag(const uint4* lds, int row, int kk, int lane) {
    const int i = lane & 15;
    const int col = (row & ~15) + 4 * (i & 3);
    const int r0 = 8 * (lane >> 5) + (i >> 2);
    const uint4* step = lds + kk * 16 * UPR;
    const i16x4 a = tr(step, r0, col);
    const i16x4 b = tr(step, r0 + 4, col);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

template <bool KMAJ, int R, int NT>
using Stage = typename std::conditional<KMAJ, StageKm<R, NT>, StageKc<R, NT>>::type;

// FP8 operand (byte codes, k contiguous): R rows x 128 k of a k tile, LDS
// [row][8 units] with the same swizzle as StageKc (128-byte rows either way).
typedef int v8i __attribute__((ext_vector_type(8)));
template <int R, int NT>
struct Stage8 {
  static constexpr int NL = (R * 8 + NT - 1) / NT;
  static __device__ __forceinline__ void direct(uint4* lds, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int rmax,
                                                int k0, int kend) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if ((R * 8) % NT != 0 && NT / 64 * i + w >= R * 8 / 64) break;
      const int P = (NT / 64 * i + w) * 64 + lane;
      const int row = P >> 3;
      const int u = (P & 7) ^ swz128(row);
      const int gr = r0 + row, kk = k0 + 16 * u;
      const uint32_t off = (kk + 16 <= kend && gr < rmax) ? (uint32_t)((long)gr * ld + kk) : OOB;
      load_lds16(rs, lds + (NT / 64 * i + w) * 64, off);
    }
  }
  // 32 bytes of tile row `row` for the 64-wide k-step ks (0, 1) and lane
  // half hf: units 4 ks + hf and 4 ks + 2 + hf.  Which k a byte stands for
  // only has to agree between the two operands: the instruction pairs byte
  // j of lane (row, half) of one with byte j of the same half of the other.
  static __device__ __forceinline__ v8i frag(const uint4* lds, int row, int ks, int hf) {
    const uint4 a = lds[row * 8 + ((4 * ks + hf) ^ swz128(row))];
    const uint4 b = lds[row * 8 + ((4 * ks + 2 + hf) ^ swz128(row))];
    v8i v;
    v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
    v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
    return v;
  }
};

// Explicit waits: the compiler's own waits know nothing of the direct
// global -> LDS copies, and a plain __syncthreads would also drain them.
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
// all but this wave's n most recent copies have landed (vector-memory loads
// retire in issue order); n is wave-uniform, at most 15
__device__ __forceinline__ void wait_loads_but(int n) {
  switch (n) {
#define WB(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    WB(1) WB(2) WB(3) WB(4) WB(5) WB(6) WB(7) WB(8) WB(9) WB(10) WB(11) WB(12) WB(13) WB(14) WB(15)
#undef WB
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
// copy instructions wave w issues for an R-row operand staged by NT threads
// (R * 8 16-byte units; the last instruction is issued only by the waves it
// reaches, as in the staging structs)
template <int R, int NT>
__device__ __forceinline__ int copies_of_wave(int w) {
  constexpr int NL = (R * 8 + NT - 1) / NT;
  int c = 0;
#pragma unroll
  for (int i = 0; i < NL; ++i) c += (NT / 64 * i + w < R * 8 / 64) ? 1 : 0;
  return c;
}

template <int TM, int TN>
struct Frags {
  bf16x8 a[TM], b[TN];
};

// ------------------------------------------------------------ MFMA kernel
// NW waves, WGM of them along M; each wave owns (BM / WGM) x (BN / (NW / WGM))
// outputs as TM x TN tiles of 32 x 32.  With 8 waves two share each SIMD, so
// one wave's MFMAs run while the other waits on LDS or the barrier.
// k-loop per 64-wide tile t: the next tile's direct copies are issued first;
// then for each 16-wide k-step the fragments of the following step are read
// from LDS while this step's MFMAs run; halfway through the last step every
// wave waits for its copies of tile t + 1 and meets the barrier, so the
// first fragments of tile t + 1 are read while the last MFMAs of tile t run.
// One output tile (tm, tn) over k in [kbeg, kend).  part == nullptr: the
// epilogue of EPI; else the raw fp32 accumulators go to part as a dense
// BM x BN tile (a partial sum for a later fixed-order reduction).
// F8 != 0: FP8 operands (F8 = 1: A and B E4M3; 2: A E5M2, B E4M3), k tiles
// of 128 bytes, one v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales)
// per 64 k; the accumulators are dequantized before the epilogue.
template <bool A_KMAJ, bool B_KMAJ, int EPI, int BM, int BN, int NW, int WGM, int F8 = 0>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int tm, int tn, int kbeg, int kend,
                                          float* __restrict__ part) {
  constexpr int NT = NW * 64;
  constexpr int WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int KK = BK / 16;
  constexpr int SA_UNITS = BM * 8, STAGE_UNITS = (BM + BN) * 8;
  // the epilogue stages SR rows x (WN + 4) floats per wave in the same LDS
  // (32 rows, or 16 when 32 would not fit in the 160 KB of a CU)
  constexpr int SR = NW * 32 * (WN + 4) * 4 <= 160 * 1024 ? 32 : 16;
  constexpr int EPI_UNITS = NW * SR * (WN + 4) / 4;
  // the fused RoPE / QK-norm epilogue stages 64-row x 256-column strips of
  // the whole tile, double-buffered, with rows padded to QKP floats
  constexpr int QKP = 260;
  constexpr int QK_UNITS = EPI == EPI_QKNORM ? 2 * 64 * QKP / 4 : 0;
  // 256 x 160 and 256 x 96 bf16 tiles keep three k-tile stages (156 and
  // 135 KB), so that two tiles' copies are in flight while the MFMAs run;
  // the others keep two
  constexpr bool PIPE3 = F8 == 0 && NW == 8 && BM == 256 && (BN == 160 || BN == 96);
  constexpr int NSTAGE = PIPE3 ? 3 : 2;
  constexpr int LDS_UNITS0 = NSTAGE * STAGE_UNITS > EPI_UNITS ? NSTAGE * STAGE_UNITS : EPI_UNITS;
  __shared__ uint4 lds[LDS_UNITS0 > QK_UNITS ? LDS_UNITS0 : QK_UNITS];
  using SA = Stage<A_KMAJ, BM, NT>;
  using SB = Stage<B_KMAJ, BN, NT>;

  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = (wave % WGM) * WM;
  const int wn = (wave / WGM) * WN;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;

  // record counts: rows x leading dimension of each operand, in bytes
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, p.b_bytes);

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  auto issue = [&](int t) {
    uint4* st = lds + (t & 1) * STAGE_UNITS;
    const int k0 = kbeg + t * BK;
    SA::direct(st, ra, p.lda, m0, p.M, k0, kend);
    SB::direct(st + SA_UNITS, rb, p.ldb, n0, p.N, k0, kend);
  };
  auto read = [&](Frags<TM, TN>& F, int t, int kk) {
    const uint4* As = lds + (t & 1) * STAGE_UNITS;
    const uint4* Bs = As + SA_UNITS;
#pragma unroll
    for (int i = 0; i < TM; ++i) F.a[i] = SA::frag(As, wm + 32 * i + lrow, kk, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) F.b[j] = SB::frag(Bs, wn + 32 * j + lrow, kk, lane);
  };

  Frags<TM, TN> F[2];
  // the explicit pipeline keeps two fragment sets live; wide 8-wave tiles
  // (64 x 160 per wave) cannot afford them and use the compiler's schedule
  constexpr bool PIPE = NW == 8 && TM * TN <= 8;
  if constexpr (F8 != 0) {
    static_assert(!A_KMAJ && !B_KMAJ, "FP8 operands are k-contiguous");
    constexpr int FA = F8 == 2 ? 1 : 0, FB = 0;  // instruction format codes: 0 E4M3, 1 E5M2
    (void)F;
    const int nk8 = kend > kbeg ? (kend - kbeg + 127) / 128 : 0;
    auto issue8 = [&](int t) {
      uint4* st = lds + (t & 1) * STAGE_UNITS;
      const int k0 = kbeg + t * 128;
      Stage8<BM, NT>::direct(st, ra, p.lda, m0, p.M, k0, kend);
      Stage8<BN, NT>::direct(st + SA_UNITS, rb, p.ldb, n0, p.N, k0, kend);
    };
    if (nk8 > 0) issue8(0);
    wait_loads();
    __syncthreads();
    for (int t = 0; t < nk8; ++t) {
      if (t + 1 < nk8) issue8(t + 1);
      const uint4* As = lds + (t & 1) * STAGE_UNITS;
      const uint4* Bs = As + SA_UNITS;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = Stage8<BM, NT>::frag(As, wm + 32 * i + lrow, ks, lhalf);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = Stage8<BN, NT>::frag(Bs, wn + 32 * j + lrow, ks, lhalf);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[j][i], FB, FA, 0, 127, 0, 127);
      }
      wait_loads();
      __syncthreads();
    }
    const float inv = p.f8_sa[2] * p.f8_sb[2];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] *= inv;
  } else if constexpr (PIPE3) {
    static_assert(TM * TN <= 8, "fragment pipeline");
    // Tile t + 2's copies go into the stage tile t - 1 used, as tile t
    // starts; at the end of tile t every wave waits only for tile t + 1
    // (tile t + 2's copies stay in flight).  Unrolled by three so that every
    // stage index is a compile-time constant.
    const int ncp = __builtin_amdgcn_readfirstlane(copies_of_wave<BM, NT>(wave) + copies_of_wave<BN, NT>(wave));
    auto issue_s = [&](int t, auto sc) __attribute__((always_inline)) {
      uint4* st = lds + decltype(sc)::value * STAGE_UNITS;
      const int k0 = kbeg + t * BK;
      SA::direct(st, ra, p.lda, m0, p.M, k0, kend);
      SB::direct(st + SA_UNITS, rb, p.ldb, n0, p.N, k0, kend);
    };
    // copy instruction c of a tile (A's first, then B's)
    constexpr int NCP = SA::NL + SB::NL;
    auto issue1 = [&](int t, auto sc, int c) __attribute__((always_inline)) {
      uint4* st = lds + decltype(sc)::value * STAGE_UNITS;
      const int k0 = kbeg + t * BK;
      if (c < SA::NL) SA::direct1(st, ra, p.lda, m0, p.M, k0, kend, c);
      else SB::direct1(st + SA_UNITS, rb, p.ldb, n0, p.N, k0, kend, c - SA::NL);
    };
    auto read_s = [&](Frags<TM, TN>& Fr, auto sc, int kk) __attribute__((always_inline)) {
      const uint4* As = lds + decltype(sc)::value * STAGE_UNITS;
      const uint4* Bs = As + SA_UNITS;
#pragma unroll
      for (int i = 0; i < TM; ++i) Fr.a[i] = SA::frag(As, wm + 32 * i + lrow, kk, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) Fr.b[j] = SB::frag(Bs, wn + 32 * j + lrow, kk, lane);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    if (nk > 0) {
      issue_s(0, S0{});
      if (nk > 1) issue_s(1, S1{});
      wait_loads_but(nk > 1 ? ncp : 0);
      block_barrier();
      read_s(F[0], S0{}, 0);
    }
    auto ktile = [&](int t, auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      using SN = std::integral_constant<int, (S + 1) % 3>;
      using SI = std::integral_constant<int, (S + 2) % 3>;
      const bool more2 = t + 2 < nk;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Frags<TM, TN>& cur = F[kk & 1];
        Frags<TM, TN>& nxt = F[(kk + 1) & 1];
        constexpr int NMF = TM * TN;
        constexpr int FIRST = NMF / 2;
        if (kk + 1 < KK) {
          read_s(nxt, sc, kk + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < NMF; ++q) {
            acc[q / TM][q % TM] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[q / TM], cur.a[q % TM], acc[q / TM][q % TM], 0, 0, 0);
            // tile t + 2's copies, one after every other MFMA of the first
            // KK - 1 steps, so that no wave stalls on a burst of them
#pragma unroll
            for (int c = 0; c < NCP; ++c) {
              if ((c * (KK - 1) * NMF) / NCP == kk * NMF + q && more2) {
                __builtin_amdgcn_sched_barrier(0);
                issue1(t + 2, SI{}, c);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int q = 0; q < FIRST; ++q)
            acc[q / TM][q % TM] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[q / TM], cur.a[q % TM], acc[q / TM][q % TM], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          // tile t + 1 has landed and every wave is done with stage S (after
          // the last tile this reads a stale stage that is never used)
          wait_loads_but(more2 ? ncp : 0);
          wait_lds();
          block_barrier();
          read_s(nxt, SN{}, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = FIRST; q < NMF; ++q)
            acc[q / TM][q % TM] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[q / TM], cur.a[q % TM], acc[q / TM][q % TM], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    for (int t = 0; t < nk; t += 3) {
      ktile(t, S0{});
      if (t + 1 < nk) ktile(t + 1, S1{});
      if (t + 2 < nk) ktile(t + 2, S2{});
    }
  } else if constexpr (PIPE) {
    if (nk > 0) {
      issue(0);
      wait_loads();
      block_barrier();
      read(F[0], 0, 0);
    }
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) issue(t + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Frags<TM, TN>& cur = F[kk & 1];
        Frags<TM, TN>& nxt = F[(kk + 1) & 1];
        constexpr int NMF = TM * TN;
        // MFMAs of this step issued before the fragment reads below: all of
        // them, except on the last step, where half of them go first and the
        // rest cover the barrier and the next tile's first reads
        constexpr int FIRST = NMF / 2;
        if (kk + 1 < KK) {
          read(nxt, t, kk + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < NMF; ++q)
            acc[q / TM][q % TM] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[q / TM], cur.a[q % TM], acc[q / TM][q % TM], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int q = 0; q < FIRST; ++q)
            acc[q / TM][q % TM] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[q / TM], cur.a[q % TM], acc[q / TM][q % TM], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          // tile t + 1 has landed and every wave is done with stage t & 1
          // (after the last tile this reads a stale stage that is never used)
          wait_loads();
          wait_lds();
          block_barrier();
          read(nxt, t + 1, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = FIRST; q < NMF; ++q)
            acc[q / TM][q % TM] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[q / TM], cur.a[q % TM], acc[q / TM][q % TM], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
    // reads and MFMAs of a tile are left to the compiler's schedule, the
    // barrier closes the tile
    if (nk > 0) issue(0);
    wait_loads();
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) issue(t + 1);
      // LLVM's igrouplp strategy 0 interleaves the LDS reads with the MFMAs;
      // measured faster with a k-major B operand (transposed reads), slower
      // with a k-contiguous one
      if constexpr (B_KMAJ) __builtin_amdgcn_iglp_opt(0);
      read(F[0], t, 0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) read(F[(kk + 1) & 1], t, kk + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[kk & 1].b[j], F[kk & 1].a[i], acc[j][i], 0, 0, 0);
      }
      wait_loads();
      __syncthreads();
    }
  }
  wait_loads();
  wait_lds();
  block_barrier();

  if constexpr (EPI == EPI_QKNORM) {
    // RoPE, then QK-norm, on the q and k heads of the tile (p.N = 3 C, head
    // dim 128: the tile's 256 columns are two heads).  Strip i of every wave
    // (rows 32 i.. of its 128) is staged into a 64 x 256 block of LDS; eight
    // threads then share each row: thread q owns the RoPE pairs 8 q .. 8 q + 7
    // of both heads (columns 8 q.. and 64 + 8 q.. of each), so the rotation is
    // thread-local, one (cos, sin) fetch serves both heads, and a head's sum
    // of squares takes three exchanges within the eight.
    static_assert(NW == 8 && WGM == 2 && BM == 256 && BN == 256, "fused RoPE / QK-norm: 256 x 256 tiles, 8 waves");
    float* eb = reinterpret_cast<float*>(lds);
    const int C3 = p.N / 3;
    const int H = C3 / 128;
    const int rr = wave * 8 + (lane >> 3);  // staged row 0..63
    const int q = lane & 7;
    int which[2];                           // 0 q, 1 k, 2 v; 3: beyond N (a last, single-head tile)
    which[0] = n0 / C3;
    which[1] = (n0 + 128) / C3;
    const bool rot = p.qk_rope && (which[0] < 2 || which[1] < 2);
    float bias[2][2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) bias[h][0][e] = bias[h][1][e] = 0.0f;
    if (p.bias) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (n0 + 128 * h >= p.N) continue;
        const bf16* b = reinterpret_cast<const bf16*>(p.bias) + n0 + 128 * h + 8 * q;
        Vec8<bf16>::load(b, bias[h][0]);
        Vec8<bf16>::load(b + 64, bias[h][1]);
      }
    }
    // (cos, sin) of the thread's 8 pairs for its row of strip i
    auto cs_row = [&](int i) -> const float4* {
      const int m = m0 + (rr >> 5) * WM + 32 * i + (rr & 31);
      const int t = (m < p.M ? m : 0) % p.qk_T;
      return reinterpret_cast<const float4*>(p.qk_cs + (long)t * 64 + 8 * q);
    };
    float4 cn[4];
    if (rot) {
      const float4* c = cs_row(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) cn[k] = c[k];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float* e = eb + (i & 1) * 64 * QKP;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(e + ((wave % WGM) * 32 + lrow) * QKP + wn + 32 * j + 8 * g + 4 * lhalf) =
              make_float4(acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]);
      wait_lds();
      block_barrier();
      const int m = m0 + (rr >> 5) * WM + 32 * i + (rr & 31);
      float v[2][2][8];  // [head][lo, hi][pair]
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float* er = e + rr * QKP + 128 * h + 64 * u + 8 * q;
          const float4 a = *reinterpret_cast<const float4*>(er);
          const float4 b = *reinterpret_cast<const float4*>(er + 4);
          v[h][u][0] = a.x + bias[h][u][0]; v[h][u][1] = a.y + bias[h][u][1];
          v[h][u][2] = a.z + bias[h][u][2]; v[h][u][3] = a.w + bias[h][u][3];
          v[h][u][4] = b.x + bias[h][u][4]; v[h][u][5] = b.y + bias[h][u][5];
          v[h][u][6] = b.z + bias[h][u][6]; v[h][u][7] = b.w + bias[h][u][7];
        }
      if (rot) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (which[h] < 2) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float4 c = cn[k];  // pairs 2 k and 2 k + 1: (cos, sin, cos, sin)
              const float l0 = v[h][0][2 * k], h0 = v[h][1][2 * k];
              const float l1 = v[h][0][2 * k + 1], h1 = v[h][1][2 * k + 1];
              v[h][0][2 * k] = fmaf(l0, c.x, -h0 * c.y);
              v[h][1][2 * k] = fmaf(h0, c.x, l0 * c.y);
              v[h][0][2 * k + 1] = fmaf(l1, c.z, -h1 * c.w);
              v[h][1][2 * k + 1] = fmaf(h1, c.z, l1 * c.w);
            }
          }
        }
        if (i + 1 < TM) {
          const float4* c = cs_row(i + 1);
#pragma unroll
          for (int k = 0; k < 4; ++k) cn[k] = c[k];
        }
      }
      if (p.qk_norm) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float ss = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) ss = fmaf(v[h][0][k], v[h][0][k], fmaf(v[h][1][k], v[h][1][k], ss));
          ss += __shfl_xor(ss, 1, 64);
          ss += __shfl_xor(ss, 2, 64);
          ss += __shfl_xor(ss, 4, 64);
          if (which[h] < 2) {
            const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + p.qk_eps);
#pragma unroll
            for (int k = 0; k < 8; ++k) { v[h][0][k] *= r; v[h][1][k] *= r; }
            if (q == 0 && m < p.M)
              p.qk_rstd[(long)which[h] * p.M * H + (long)m * H + ((n0 + 128 * h) % C3) / 128] = r;
          }
        }
      }
      if (m < p.M) {
        bf16* o = reinterpret_cast<bf16*>(p.out) + (long)m * p.ldc + n0 + 8 * q;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (n0 + 128 * h >= p.N) continue;
          Vec8<bf16>::store(o + 128 * h, v[h][0]);
          Vec8<bf16>::store(o + 128 * h + 64, v[h][1]);
        }
      }
    }
    return;
  }

  // Epilogue through LDS (free after the barrier above): each wave writes
  // one 32-row strip of its accumulators (lane: row lrow, columns
  // 32 j + 8 g + 4 lhalf + e) and reads it back as 8-column row vectors, so
  // global reads and writes of the epilogue are contiguous 16-byte vectors.
  constexpr int PITCH = WN + 4;           // floats per staged row
  constexpr int LPR = WN / 8;             // 8-column vectors (lanes) per row in the read-back
  static_assert((SR * LPR) % 64 == 0, "read-back passes must cover whole rows");
  static_assert(EPI != EPI_XENT_STATS || (64 % LPR == 0 && SR == 32), "row reductions need a row's lanes in one pass");
  float* ep = reinterpret_cast<float*>(lds) + wave * (SR * PITCH);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
  for (int h = 0; h < 32 / SR; ++h) {
    if (SR == 32 || (lrow / SR) == h) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(ep + (lrow - h * SR) * PITCH + 32 * j + 8 * g + 4 * lhalf) =
              make_float4(acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    // resid / GELU'(u) row vectors of every pass are fetched before the first
    // store, so their latencies overlap (the compiler may not move a load
    // across a store to the output, which could alias it)
    constexpr int NPASS = SR * LPR / 64;
    constexpr bool PRE = EPI == EPI_STORE || EPI == EPI_GELU_BWD;
    const bf16* pre_src = nullptr;
    long pre_ld = 0;
    if constexpr (EPI == EPI_STORE) { pre_src = reinterpret_cast<const bf16*>(p.resid); pre_ld = p.ldr; }
    if constexpr (EPI == EPI_GELU_BWD) { pre_src = reinterpret_cast<const bf16*>(p.aux); pre_ld = p.ldaux; }
    uint4 pre[PRE ? NPASS : 1];
    if constexpr (PRE) {
      if (pre_src && !part) {
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
          const int item = pass * 64 + lane;
          const int m = m0 + wm + 32 * i + h * SR + item / LPR;
          const int n = n0 + wn + (item % LPR) * 8;
          pre[pass] = (m < p.M && n + 8 <= p.N) ? *reinterpret_cast<const uint4*>(pre_src + (long)m * pre_ld + n)
                                                : make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int item = pass * 64 + lane;
      const int row = h * SR + item / LPR;  // row within the 32-row strip
      const int col = (item % LPR) * 8;
      const float* er = ep + (row - h * SR) * PITCH;
      float v[8];
      const float4 a = *reinterpret_cast<const float4*>(er + col);
      const float4 b = *reinterpret_cast<const float4*>(er + col + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      const int m = m0 + wm + 32 * i + row;
      const int n = n0 + wn + col;
      if constexpr (EPI == EPI_XENT_STATS) {
        // (max, sum exp) of this row over the wave's WN columns; LPR lanes share a row
        const int tg = (m < p.M) ? p.tgt[m] - p.col_offset : -1;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (n + e < p.N) mx = fmaxf(mx, v[e]);
          if (n + e == tg) p.ztgt[m] = v[e];
        }
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float sm = 0.0f;
        if (mx != -INFINITY) {
          const float ms = mx * LOG2E;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < p.N) sm += exp2f(fmaf(v[e], LOG2E, -ms));
        }
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 64);
        if (m < p.M && lane % LPR == 0)
          p.part[(long)m * p.part_ld + p.part_off + (n0 + wn) / WN] = make_float2(mx, sm);
      } else {
        if (part) {
          float* d = part + (long)(m - m0) * BN + (n - n0);
          reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
          reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          epiW<bf16, EPI, 8>(p, m, n, v, PRE && pre_src, pre[PRE ? pass : 0]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool A_KMAJ, bool B_KMAJ, int EPI, int BM, int BN, int NW, int WGM, int F8 = 0>
__global__ __launch_bounds__(NW * 64, 1) void gemm_mfma(GemmParams p) {
  int tm, tn;
  tile_coords(p, blockIdx.x, gridDim.x, tm, tn);
  const int kbeg = blockIdx.z * p.k_split;
  gemm_tile<A_KMAJ, B_KMAJ, EPI, BM, BN, NW, WGM, F8>(p, tm, tn, kbeg, min(p.K, kbeg + p.k_split), nullptr);
}

// Several independent problems of one kind in a single launch: blocks
// [start[q], start[q + 1]) cover the tiles of problem q.
struct GemmGroup {
  GemmParams p[GEMM_GROUP_MAX];
  int start[GEMM_GROUP_MAX + 1];
  int count;
};

// Grouped problems that share K, as "data-parallel + stream-K": with T
// tiles over G blocks, block b first computes whole tiles b, b + G, ...
// (R = T / G of them); the k-steps of the remaining T - R G tiles are then
// split evenly over the G blocks, each writing its piece of a tile as an fp32
// partial into slot (tile, piece) for streamk_fixup to add in order.
struct StreamKPlan {
  int G;          // blocks
  int R;          // whole tiles per block
  int nk;         // k units per tile
  int ku;         // k elements per unit (one k tile: BK, or 128 for FP8 codes)
  int rem;        // tiles left for the split phase
  int S;          // partial slots per split tile
  float* part;    // [rem][S][BM * BN]
  bool wide;      // 256 x 320 tiles in a single round (R = 1, rem = 0)
};

__host__ __device__ inline long sk_units_begin(const StreamKPlan& k, int b) {
  return (long)b * k.rem * k.nk / k.G;
}
// the block whose split-phase range holds unit u
__host__ __device__ inline int sk_block_of(const StreamKPlan& k, long u) {
  int b = (int)(u * k.G / ((long)k.rem * k.nk));
  while (b + 1 < k.G && sk_units_begin(k, b + 1) <= u) ++b;
  while (b > 0 && sk_units_begin(k, b) > u) --b;
  return b;
}

template <int BM, int BN>
__device__ __forceinline__ void group_tile(const GemmGroup& g, int tile, int& q, int& tm, int& tn) {
  q = 0;
#pragma unroll
  for (int i = 1; i < GEMM_GROUP_MAX; ++i)
    if (i < g.count && tile >= g.start[i]) q = i;
  tile_coords(g.p[q], tile - g.start[q], g.start[q + 1] - g.start[q], tm, tn);
}

template <bool A_KMAJ, bool B_KMAJ, int EPI, int BM, int BN, int NW, int WGM, int F8 = 0>
__global__ __launch_bounds__(NW * 64, 1) void gemm_streamk(GemmGroup g, StreamKPlan k) {
  const int b = blockIdx.x;
  int q, tm, tn;
  for (int r = 0; r < k.R; ++r) {
    group_tile<BM, BN>(g, r * k.G + b, q, tm, tn);
    gemm_tile<A_KMAJ, B_KMAJ, EPI, BM, BN, NW, WGM, F8>(g.p[q], tm, tn, 0, g.p[q].K, nullptr);
    block_barrier();  // the epilogue's LDS staging is done before the next prologue
  }
  if (k.rem == 0) return;
  const long u1 = sk_units_begin(k, b + 1);
  for (long u = sk_units_begin(k, b); u < u1;) {
    const int rt = (int)(u / k.nk);                 // split-phase tile
    const int k0 = (int)(u % k.nk);
    const int k1 = (int)min((long)k.nk, k0 + (u1 - u));
    group_tile<BM, BN>(g, k.R * k.G + rt, q, tm, tn);
    const GemmParams& p = g.p[q];
    float* part = nullptr;
    if (k0 != 0 || k1 != k.nk) {
      const int first = sk_block_of(k, (long)rt * k.nk);
      part = k.part + ((long)rt * k.S + (b - first)) * (BM * BN);
    }
    gemm_tile<A_KMAJ, B_KMAJ, EPI, BM, BN, NW, WGM, F8>(p, tm, tn, k0 * k.ku, min(p.K, k1 * k.ku), part);
    block_barrier();
    u += k1 - k0;
  }
}

// Grouped problems in one round of whole tiles, one tile per block.
template <bool A_KMAJ, bool B_KMAJ, int EPI, int BM, int BN, int NW, int WGM, int F8 = 0>
__global__ __launch_bounds__(NW * 64, 1) void gemm_group_dp(GemmGroup g) {
  int q, tm, tn;
  group_tile<BM, BN>(g, blockIdx.x, q, tm, tn);
  gemm_tile<A_KMAJ, B_KMAJ, EPI, BM, BN, NW, WGM, F8>(g.p[q], tm, tn, 0, g.p[q].K, nullptr);
}

// Adds the partial slots of each split-phase tile in piece order (fixed
// order: bitwise reproducible) and writes the fp32 result (+= when the
// problem accumulates).  One block per (tile, 256 x 8-column group).
template <int BM, int BN>
__global__ __launch_bounds__(256) void streamk_fixup(GemmGroup g, StreamKPlan k) {
  const int rt = blockIdx.y;
  const int first = sk_block_of(k, (long)rt * k.nk);
  const int last = sk_block_of(k, (long)(rt + 1) * k.nk - 1);
  if (first == last) return;  // one block computed it whole
  int q, tm, tn;
  group_tile<BM, BN>(g, k.R * k.G + rt, q, tm, tn);
  const GemmParams& p = g.p[q];
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;  // element within the tile
  if (e >= BM * BN) return;
  const int r = e / BN, c = e % BN;
  const int m = tm * BM + r, n = tn * BN + c;
  if (m >= p.M || n >= p.N) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j <= last - first; ++j) {
    // a block with an empty unit range (rem * nk < G) wrote no slot; every
    // other block in first..last holds a piece of this tile
    if (sk_units_begin(k, first + j) == sk_units_begin(k, first + j + 1)) continue;
    const float4 v = *reinterpret_cast<const float4*>(k.part + ((long)rt * k.S + j) * (BM * BN) + e);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  float* o = reinterpret_cast<float*>(p.out) + (long)m * p.ldc + n;
  const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
  for (int t = 0; t < 4; ++t)
    if (n + t < p.N) o[t] = p.accumulate ? o[t] + a4[t] : a4[t];
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
    epiW<T, EPI, 4>(p, m0 + ty * 4 + i, n0 + tx * 4, v);
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
  const long t160 = (long)cdiv(d.M, 256) * cdiv(d.N, 160);
  const long t320 = (long)cdiv(d.M, 256) * cdiv(d.N, 320);
  // whole rounds of the 256 CUs: 256 x 320 when it fills them exactly and
  // 256 x 256 would leave a partial round (e.g. N = 5120, M = 8192)
  const bool r320 = d.N % 320 == 0 && t320 >= 256 && t320 % 256 == 0 && t256 % 256 != 0;
  // 256 x 192 (bf16, A k-contiguous, B either way; store, GELU, GELU' and
  // fp32 epilogues) where it fills the CUs in whole rounds and 256 x 256
  // would not: the GPT-2 width's N = 3072 at M = 8192 (FC forward, proj
  // input gradient) and N = 768 at M = 16384 (the LM head's input gradient
  // among them; a 128 x 192 tile for N = 768 at M = 8192 measured no faster
  // than 128 x 128)
  const long t192 = d.N % 192 == 0 ? (long)cdiv(d.M, 256) * (d.N / 192) : 0;
  const bool r192 = t192 > 0 && !d.a_kmaj && !d.f8_sa &&
                    (d.epi == EPI_STORE || d.epi == EPI_GELU || d.epi == EPI_GELU_BWD || d.epi == EPI_F32) &&
                    t192 % 256 == 0 && t256 % 256 != 0;
  // fp32-output products with both operands k-major (weight-gradient form,
  // long K): 256 x 192 when the tiles, split along K, fill the 256 CUs
  // exactly (the GPT-2 LM head's dW: 128 tiles, two K halves)
  const bool k192 = t192 > 0 && d.a_kmaj && d.b_kmaj && !d.f8_sa && d.epi == EPI_F32 && 256 % t192 == 0 &&
                    d.K / (256 / t192) >= 1024;
  // 256 x 96 (8 waves of 32 x 96, k-contiguous bf16, store epilogue) where
  // it fills the CUs in whole rounds and neither 256 x 256 nor 256 x 192
  // would: at the GPT-2 width and M = 8192, the N = 768 products (one round)
  // and the QKV forward (N = 2304: three rounds, against 1.125 of 256 x 256)
  const bool r96 = d.N % 96 == 0 && !d.a_kmaj && !d.b_kmaj && !d.f8_sa && d.epi == EPI_STORE &&
                   (long)cdiv(d.M, 256) * (d.N / 96) % 256 == 0 && t256 % 256 != 0 &&
                   !(t192 > 0 && t192 % 256 == 0);
  if (d.epi == EPI_XENT_STATS || d.epi == EPI_QKNORM) { pl.BMv = 256; pl.BNv = 256; }
  else if (r96) { pl.BMv = 256; pl.BNv = 96; }
  else if (r320 && d.epi != EPI_F32) { pl.BMv = 256; pl.BNv = 320; }
  else if (r192 || k192) { pl.BMv = 256; pl.BNv = 192; }
  else if (t256 >= 240) { pl.BMv = 256; pl.BNv = 256; }
  else if (d.N % 160 == 0 && t160 >= 240 && t160 % 256 <= 16) { pl.BMv = 256; pl.BNv = 160; }
  else { pl.BMv = 128; pl.BNv = 128; }
  const long tiles = (long)cdiv(d.M, pl.BMv) * cdiv(d.N, pl.BNv);
  // split until the blocks cover the 256 CUs once (each split adds an fp32
  // partial of the whole output to write and reduce)
  const long slots = 256;
  pl.splits = 1;
  if (d.epi == EPI_F32) {
    // weight gradients: small output, long K -> split K (fp32 partials,
    // fixed-order reduce) until every CU has work
    while (tiles * pl.splits < slots && d.K / (pl.splits * 2) >= 256) pl.splits *= 2;
  }
  pl.k_split = cdiv(cdiv(d.K, pl.splits), BK) * BK;
  pl.splits = cdiv(d.K, pl.k_split);
  return pl;
}

// 256 x 256 tiles run 8 waves (two per SIMD, 128 x 64 each, or 64 x 128 for
// the fused RoPE / QK-norm epilogue, whose waves each hold one head); in the
// LM-head statistics a wave's 64 columns make one (max, sum exp) partial.
// 128 x 128 tiles run 4 waves of 64 x 64.
template <bool AK, bool BKm, int EPI, int BMv, int BNv, int F8 = 0>
hipError_t go_mfma(const GemmParams& p, int splits, hipStream_t s) {
  dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
  if constexpr (BMv == 256)
    hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, BMv, BNv, 8, 2, F8>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, BMv, BNv, 4, 2, F8>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// Wide tiles: 256 x 320 (8 waves of 64 x 160) where they fill the CUs in
// whole rounds and 256 x 256 would not; 256 x 160 (N a multiple of 160, e.g.
// 1280 = 8 x 160 with M = 8192: exactly one tile per CU) as 8 waves of
// 32 x 160, two per SIMD.
template <bool AK, bool BKm, int EPI, int F8 = 0>
hipError_t go_mfma_tiles(const GemmParams& p, const Plan& pl, hipStream_t s) {
  if (pl.BMv == 256 && pl.BNv == 256) return go_mfma<AK, BKm, EPI, 256, 256, F8>(p, pl.splits, s);
  if (pl.BNv == 320) {
    // 8 waves of 64 x 160
    if constexpr (EPI == EPI_XENT_STATS || EPI == EPI_QKNORM || EPI == EPI_F32) {
      return hipErrorInvalidValue;
    } else {
      dim3 grid(p.tiles_m * p.tiles_n, 1, pl.splits);
      hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, 256, 320, 8, 4, F8>), grid, dim3(512), 0, s, p);
      return hipGetLastError();
    }
  }
  if (pl.BNv == 192) {
    // 8 waves of 64 x 96
    if constexpr (F8 == 0 && (AK ? (BKm && EPI == EPI_F32)
                                 : (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_GELU_BWD || EPI == EPI_F32))) {
      dim3 grid(p.tiles_m * p.tiles_n, 1, pl.splits);
      hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, 256, 192, 8, 4, F8>), grid, dim3(512), 0, s, p);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (pl.BNv == 96) {
    // 8 waves of 32 x 96
    if constexpr (F8 == 0 && !AK && !BKm && EPI == EPI_STORE) {
      dim3 grid(p.tiles_m * p.tiles_n, 1, pl.splits);
      hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, 256, 96, 8, 8, F8>), grid, dim3(512), 0, s, p);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (pl.BNv == 160) {
    if constexpr (EPI == EPI_XENT_STATS || EPI == EPI_QKNORM) {
      return hipErrorInvalidValue;
    } else {
      dim3 grid(p.tiles_m * p.tiles_n, 1, pl.splits);
      hipLaunchKernelGGL((gemm_mfma<AK, BKm, EPI, 256, 160, 8, 8, F8>), grid, dim3(512), 0, s, p);
      return hipGetLastError();
    }
  }
  return go_mfma<AK, BKm, EPI, 128, 128, F8>(p, pl.splits, s);
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
  p.part_off = d.part_off; p.ztgt = d.ztgt; p.lse = d.lse; p.scale = d.scale; p.roww = d.roww;
  p.qk_cs = d.qk_cs; p.qk_rstd = d.qk_rstd; p.qk_T = d.qk_T; p.qk_rope = d.qk_rope; p.qk_norm = d.qk_norm;
  p.qk_eps = d.qk_eps;
  p.f8_sa = d.f8_sa; p.f8_sb = d.f8_sb;
  return p;
}

// ---------------------------------------------------------------- transpose
__global__ __launch_bounds__(256) void transpose_bf16_k(TransposeJobs J) { transpose_block(J, blockIdx.x); }

}  // namespace

int xent_part_cols() { return 64; }

size_t gemm_split_scratch_bytes(const GemmDesc& d, int dtype) {
  if (dtype != 1 || d.epi != EPI_F32) return 0;
  // sizes only: the MFMA path may take any such problem
  Plan pl = plan_mfma(d);
  if (pl.splits <= 1) return 0;
  return align256((size_t)pl.splits * d.M * d.N * sizeof(float));
}

// Extent in bytes of an operand stored [rows][ld] whose last row is read up
// to `cols` elements; 0 if the MFMA path cannot take it (the contiguous
// extent or leading dimension is not a multiple of 8, the base is not
// 16-byte aligned, or offsets would not fit the 31-bit buffer range).
static uint32_t operand_bytes(const void* p, long rows, long ld, long cols) {
  if (rows <= 0 || cols % 8 || ld % 8 || (reinterpret_cast<uintptr_t>(p) & 15)) return 0;
  const long bytes = ((rows - 1) * ld + cols) * 2;
  if (bytes <= 0 || bytes >= (1L << 31)) return 0;
  return (uint32_t)bytes;
}

static bool mfma_ok(const GemmDesc& d, uint32_t& ab, uint32_t& bb) {
  ab = d.a_kmaj ? operand_bytes(d.A, d.K, d.lda, d.M) : operand_bytes(d.A, d.M, d.lda, d.K);
  bb = d.b_kmaj ? operand_bytes(d.B, d.K, d.ldb, d.N) : operand_bytes(d.B, d.N, d.ldb, d.K);
  return ab && bb && d.K > 0;
}

hipError_t launch_gemm(const GemmDesc& d, int dtype, void* ws, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  GemmParams p = make_params(d);
  uint32_t ab = 0, bb = 0;
  if (dtype == 1 && mfma_ok(d, ab, bb)) {
    Plan pl = plan_mfma(d);
    p.tiles_m = cdiv(d.M, pl.BMv);
    p.tiles_n = cdiv(d.N, pl.BNv);
    p.k_split = pl.k_split;
    p.a_bytes = ab;
    p.b_bytes = bb;
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
      case EPI_QKNORM:
        if (!ak && !bk && d.N % 384 == 0) e = go_mfma<false, false, EPI_QKNORM, 256, 256>(p, pl.splits, s);
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
  if (dtype == 1) {
    // bf16 operands the MFMA path cannot take (odd extents): SIMT kernel
    p.k_split = d.K > 0 ? d.K : 0;
    const bool ak = d.a_kmaj, bk = d.b_kmaj;
    if (d.epi == EPI_F32 && ak && bk) return go_simt<bf16, true, true, EPI_F32>(p, 1, s);
    if (d.epi == EPI_F32 && !ak && bk) return go_simt<bf16, false, true, EPI_F32>(p, 1, s);
    return hipErrorInvalidValue;
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

// FP8 GEMMs: the MFMA path's tile plan with 128-element k tiles for split-K.
static Plan plan_fp8(const GemmDesc& d) {
  Plan pl = plan_mfma(d);
  pl.k_split = cdiv(cdiv(d.K, pl.splits), 128) * 128;
  pl.splits = cdiv(d.K, pl.k_split);
  return pl;
}

size_t gemm_fp8_split_scratch_bytes(const GemmDesc& d) {
  if (d.epi != EPI_F32) return 0;
  const Plan pl = plan_fp8(d);
  return pl.splits > 1 ? align256((size_t)pl.splits * d.M * d.N * sizeof(float)) : 0;
}

hipError_t launch_gemm_fp8(const GemmDesc& d, int mode, void* ws, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  if (d.a_kmaj || d.b_kmaj || d.K <= 0 || d.K % 16 || d.lda % 16 || d.ldb % 16 || !d.f8_sa || !d.f8_sb)
    return hipErrorInvalidValue;
  const long ab = (long)(d.M - 1) * d.lda + d.K, bb = (long)(d.N - 1) * d.ldb + d.K;
  if (ab >= (1L << 31) || bb >= (1L << 31)) return hipErrorInvalidValue;
  GemmParams p = make_params(d);
  const Plan pl = plan_fp8(d);
  p.tiles_m = cdiv(d.M, pl.BMv);
  p.tiles_n = cdiv(d.N, pl.BNv);
  p.k_split = pl.k_split;
  p.a_bytes = (uint32_t)ab;
  p.b_bytes = (uint32_t)bb;
  const bool split = pl.splits > 1;
  if (split) {
    p.out = ws; p.ldc = d.N; p.accumulate = 0; p.split_stride = (long)d.M * d.N;
  }
  hipError_t e = hipErrorInvalidValue;
  if (mode == 1) {
    switch (d.epi) {
      case EPI_STORE: e = go_mfma_tiles<false, false, EPI_STORE, 1>(p, pl, s); break;
      case EPI_GELU: e = go_mfma_tiles<false, false, EPI_GELU, 1>(p, pl, s); break;
      case EPI_QKNORM:
        if (d.N % 384 == 0) e = go_mfma<false, false, EPI_QKNORM, 256, 256, 1>(p, pl.splits, s);
        break;
      default: break;
    }
  } else if (mode == 2) {
    switch (d.epi) {
      case EPI_STORE: e = go_mfma_tiles<false, false, EPI_STORE, 2>(p, pl, s); break;
      case EPI_GELU_BWD: e = go_mfma_tiles<false, false, EPI_GELU_BWD, 2>(p, pl, s); break;
      case EPI_F32: e = go_mfma_tiles<false, false, EPI_F32, 2>(p, pl, s); break;
      default: break;
    }
  }
  if (e != hipSuccess) return e;
  if (split) {
    const long total = (long)d.M * d.N;
    int blocks = (int)std::min<long>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, s, (const float*)ws, pl.splits, (long)d.M * d.N,
                       d.M, d.N, (float*)d.out, d.ldc, d.accumulate);
    e = hipGetLastError();
  }
  return e;
}

// Plan of a weight-gradient group.  When the group's 256 x 320 tiles
// fit one round of SK_BLOCKS blocks (the CU count of an MI355X) and fill at
// least 7/8 of it, one block per whole tile (plan.wide): no split phase, no
// partials, no fixup, and 10% fewer operand bytes per FLOP than 256 x 256
// (d20: 240 tiles, 318 against 335 us for the 256 x 256 stream-K launch with
// its fixup).  Otherwise stream-K over 256 x 256 tiles.  Returns false when
// the problems do not qualify (bf16 MFMA operands, both k-major, fp32
// output, one K that is a multiple of BK).
constexpr int SK_BLOCKS = 256;
// fp8: FP8 codes (dY in E5M2 times X in E4M3, both with k = tokens
// contiguous, launch_gemm_fp8's operand rules), in 128-element k units;
// otherwise bf16 with both operands k-major, in BK-element units
static bool streamk_plan(const GemmDesc* d, int n, int dtype, bool fp8, GemmGroup& g, StreamKPlan& k,
                         size_t& scratch) {
  if (n <= 0 || n > GEMM_GROUP_MAX || dtype != 1) return false;
  const int K = d[0].K;
  if (K <= 0 || K % (fp8 ? 16 : BK)) return false;
  bool wide = true;
  {
    long t320 = 0;
    for (int i = 0; i < n; ++i) t320 += (long)cdiv(d[i].M, 256) * cdiv(d[i].N, 320);
    if (t320 > SK_BLOCKS || 8 * t320 < 7L * SK_BLOCKS) wide = false;
  }
  g = GemmGroup{};
  g.count = n;
  int total = 0;
  for (int i = 0; i < n; ++i) {
    uint32_t ab = 0, bb = 0;
    if (d[i].epi != EPI_F32 || d[i].K != K || d[i].M <= 0 || d[i].N <= 0) return false;
    if (fp8) {
      if (d[i].a_kmaj || d[i].b_kmaj || d[i].lda % 16 || d[i].ldb % 16) return false;
      const long a = (long)(d[i].M - 1) * d[i].lda + K, b = (long)(d[i].N - 1) * d[i].ldb + K;
      if (a >= (1L << 31) || b >= (1L << 31)) return false;
      ab = (uint32_t)a;
      bb = (uint32_t)b;
    } else if (!d[i].a_kmaj || !d[i].b_kmaj || !mfma_ok(d[i], ab, bb)) {
      return false;
    }
    GemmParams p = make_params(d[i]);
    p.tiles_m = cdiv(d[i].M, 256);
    p.tiles_n = cdiv(d[i].N, wide ? 320 : 256);
    p.k_split = K;
    p.a_bytes = ab;
    p.b_bytes = bb;
    g.p[i] = p;
    g.start[i] = total;
    total += p.tiles_m * p.tiles_n;
  }
  for (int i = n; i <= GEMM_GROUP_MAX; ++i) g.start[i] = total;
  k = StreamKPlan{};
  k.wide = wide;
  k.G = wide ? total : SK_BLOCKS;
  k.R = total / k.G;
  k.rem = total % k.G;
  k.ku = fp8 ? 128 : BK;
  k.nk = cdiv(K, k.ku);
  k.S = 1;
  for (int rt = 0; rt < k.rem; ++rt)
    k.S = std::max(k.S, sk_block_of(k, (long)(rt + 1) * k.nk - 1) - sk_block_of(k, (long)rt * k.nk) + 1);
  scratch = k.rem ? align256((size_t)k.rem * k.S * 256 * 256 * sizeof(float)) : 0;
  return true;
}

size_t gemm_group_scratch_bytes(const GemmDesc* d, int n, int dtype) {
  GemmGroup g;
  StreamKPlan k;
  size_t need = 0;
  if (streamk_plan(d, n, dtype, false, g, k, need)) return need;
  size_t m = 0;
  for (int i = 0; i < n; ++i) m = std::max(m, gemm_split_scratch_bytes(d[i], dtype));
  return m;
}

size_t gemm_group_fp8_scratch_bytes(const GemmDesc* d, int n) {
  GemmGroup g;
  StreamKPlan k;
  size_t need = 0;
  if (streamk_plan(d, n, 1, true, g, k, need)) return need;
  size_t m = 0;
  for (int i = 0; i < n; ++i) m = std::max(m, gemm_fp8_split_scratch_bytes(d[i]));
  return m;
}

// the stream-K kernel and, when tiles were split, the fixup
template <bool AK, bool BKm, int F8>
static hipError_t run_streamk(const GemmGroup& g, StreamKPlan& k, void* ws, hipStream_t s) {
  k.part = static_cast<float*>(ws);
  if (k.wide) {
    hipLaunchKernelGGL((gemm_group_dp<AK, BKm, EPI_F32, 256, 320, 8, 4, F8>), dim3(k.G), dim3(512), 0, s, g);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_streamk<AK, BKm, EPI_F32, 256, 256, 8, 2, F8>), dim3(k.G), dim3(512), 0, s, g, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || k.rem == 0) return e;
  hipLaunchKernelGGL((streamk_fixup<256, 256>), dim3(256 * 256 / 1024, k.rem), dim3(256), 0, s, g, k);
  return hipGetLastError();
}

hipError_t launch_gemm_group(const GemmDesc* d, int n, int dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  GemmGroup g;
  StreamKPlan k;
  size_t need = 0;
  if (streamk_plan(d, n, dtype, false, g, k, need) && (need == 0 || (ws && ws_bytes >= need)))
    return run_streamk<true, true, 0>(g, k, ws, s);
  // otherwise one launch per problem
  for (int i = 0; i < n; ++i) {
    hipError_t e = launch_gemm(d[i], dtype, ws, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_group_fp8(const GemmDesc* d, int n, void* ws, size_t ws_bytes, hipStream_t s) {
  for (int i = 0; i < n; ++i)
    if (!d[i].f8_sa || !d[i].f8_sb) return hipErrorInvalidValue;
  GemmGroup g;
  StreamKPlan k;
  size_t need = 0;
  if (streamk_plan(d, n, 1, true, g, k, need) && (need == 0 || (ws && ws_bytes >= need)))
    return run_streamk<false, false, 2>(g, k, ws, s);
  for (int i = 0; i < n; ++i) {
    hipError_t e = launch_gemm_fp8(d[i], 2, ws, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_transpose(const TransposeDesc* d, int n, hipStream_t s) {
  if (n <= 0 || n > TRANSPOSE_MAX) return hipErrorInvalidValue;
  TransposeJobs J{};
  if (make_transpose_jobs(d, n, J) == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_k, dim3(J.start[n]), dim3(256), 0, s, J);
  return hipGetLastError();
}
