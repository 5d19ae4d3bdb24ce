// Causal self-attention forward/backward, RoPE + QK-norm, and the
// backward's row-dot preprocessing.
//
// Math ("nanoGPT — Karpathy's minimal GPT pretraining repo", model.py,
// CausalSelfAttention: per head S = q k^T / sqrt(D), future positions
// masked, P = softmax(S), O = P v; the nanochat-d20 form applies RoPE and a
// parameter-free RMS QK-norm to q and k first).
//
// bf16 MFMA kernels (head_dim 64 or 128), wave64, v_mfma_f32_32x32x16_bf16:
//  * forward: a workgroup owns 128 queries of one (batch, head), one wave per
//    32 queries; K and V tiles of 64 keys are staged in LDS (double buffer).
//    Each wave computes S^T = K Q^T so that a lane owns one query and its
//    softmax statistics stay in the lane (one cross-half exchange per
//    reduction); P^T is fed straight from the accumulators as the B operand
//    of O^T = V^T P^T.  Online softmax in the log2 domain; fully masked
//    tiles are skipped per wave, the causal mask is applied only to tiles
//    that cross the diagonal; log-sum-exp is saved for the backward.
//  * backward: two passes, no floating-point atomics (bitwise
//    deterministic).  dK/dV: a workgroup owns 128 keys, loops over query
//    tiles, recomputes P from the saved log-sum-exp, accumulates
//    dV^T = dO^T P and dK^T = Q^T dS.  dQ: a workgroup owns 128 queries,
//    loops over key tiles, accumulates dQ^T = K^T dS^T.
//  * MFMA k-slot order: within a 16-wide reduction step, lane half h and
//    slot e of both operands stand for the same reduction index
//    16 ks + 4 h + e (slots 0..3) or 16 ks + 8 + 4 h + e (slots 4..7), which
//    is where a 32x32 accumulator keeps its rows; operands read from LDS
//    use the same mapping.
// SIMT kernels cover fp32 storage and other head dims (any D <= 128).
#include <type_traits>

#include "kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 u4_bf8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 ld16(const bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// Raw buffer loads over one (batch, head) slice: rows at or beyond the
// record count read as zeros, so tile loads need no branches.
constexpr uint32_t OOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// rsrc over rows [0, T) of a [T][ld] bf16 slice whose rows hold D used elements
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const bf16* base, int T, long ld, int D) {
  return make_rsrc(base, ((long)(T - 1) * ld + D) * 2);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
// Pack accumulator registers 4g0..4g0+3 and 4g0+4..4g0+7 of a 32x32 tile as
// the 8 bf16 k-slots of a B operand.
__device__ __forceinline__ bf16x8 pack_slots(const float* p, int g0) {
  uint4 u;
  u.x = pack2(p[4 * g0 + 0], p[4 * g0 + 1]);
  u.y = pack2(p[4 * g0 + 2], p[4 * g0 + 3]);
  u.z = pack2(p[4 * g0 + 4], p[4 * g0 + 5]);
  u.w = pack2(p[4 * g0 + 6], p[4 * g0 + 7]);
  return u4_bf8(u);
}

// ---------------------------------------------------------------------------
// LDS tiles: 64 rows x D bf16, row-major, 16-byte unit u of row r stored at
// u ^ f(r).  The swizzle keeps both access patterns free of bank conflicts
// on a 64-bank LDS: 16-byte fragment reads of 16 consecutive rows, and
// ds_read_b64_tr_b16 reads (4 aligned rows x 16 or 32 columns).
//   256-byte rows (D = 128): f(r) = ((r & 3) << 2) | ((r >> 2) & 3)
//   128-byte rows (D = 64):  f(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
// A tile serves as an MFMA A operand two ways:
//   row_frag: rows of the tile, 8 consecutive columns per lane (16 ks + 8 hf);
//   tr_frag:  columns of the tile (the transposed matrix), via the gfx950
//             transpose read: within a 16-lane group, lane i receives element
//             i % 4 of the 4-element vectors addressed by lanes 4k + i / 4
//             (k = 0..3), so when those lanes address rows j0 + k at column
//             D0 + 4 (i % 4), lane i gets rows j0..j0+3 of column D0 + i.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int upos(int r, int u) { return r * (D / 8) + (u ^ swz<D>(r)); }

template <int D>
struct RowTile {
  static constexpr int KU = D / 8;
  static constexpr int PER = 64 * KU / 256;
  uint4 v[PER];
  // rows r0 .. r0 + 63 of the slice; rows >= T read as zeros
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, long ld, int r0, int T) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = threadIdx.x + 256 * i;
      const int r = r0 + u / KU, c = u % KU;
      v[i] = bload(rs, r < T ? (uint32_t)(((long)r * ld + 8 * c) * 2) : OOB);
    }
  }
  __device__ __forceinline__ void store(uint4* s) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = threadIdx.x + 256 * i;
      s[upos<D>(u / KU, u % KU)] = v[i];
    }
  }
  // Asynchronous global -> LDS copy of rows r0 .. r0 + 63 (no registers):
  // wave w's instruction i fills physical units P = (4 i + w) * 64 + lane,
  // i.e. row P / KU, slot P % KU, which holds logical unit slot ^ f(row);
  // lane L's 16 bytes land at the wave-uniform base + 16 L, and rows >= T
  // (out-of-range offsets) arrive as zeros.
  // the same copy spread over NW waves (NW * 64 threads)
  template <int NW>
  static __device__ __forceinline__ void direct_by(uint4* s, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int T) {
    static_assert((64 * KU) % (64 * NW) == 0, "whole copies per wave");
    constexpr int N = 64 * KU / (64 * NW);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int P = (NW * i + w) * 64 + lane;
      const int row = P / KU;
      const int u = (P % KU) ^ swz<D>(row);
      const int r = r0 + row;
      const uint32_t off = r < T ? (uint32_t)(((long)r * ld + 8 * u) * 2) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(s + (NW * i + w) * 64),
                                               16, off, 0, 0, 0);
    }
  }
  static __device__ __forceinline__ void direct(uint4* s, __amdgpu_buffer_rsrc_t rs, long ld, int r0, int T) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int P = (4 * i + w) * 64 + lane;
      const int row = P / KU;
      const int u = (P % KU) ^ swz<D>(row);
      const int r = r0 + row;
      const uint32_t off = r < T ? (uint32_t)(((long)r * ld + 8 * u) * 2) : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(s + (4 * i + w) * 64),
                                               16, off, 0, 0, 0);
    }
  }
};

// Waits on the vector-memory counter through the s_waitcnt builtin rather
// than inline asm, so that the compiler's own wait insertion sees them and
// adds no second, stricter wait before the LDS reads of a landed tile.
// Encoding (gfx9): vmcnt in bits 3:0, expcnt 6:4 and lgkmcnt 11:8 left at
// their maxima (no wait).
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Workgroup barrier for LDS data: this wave's LDS accesses complete, then
// s_barrier.  Global -> LDS copies in flight stay in flight (__syncthreads
// would also wait for those); the "memory" clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// all but the N (< 16) most recently issued vector-memory operations have retired
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Sum / max of v over the lane pair (l, l ^ 32), returned to both lanes.
// v_permlane32_swap exchanges the upper half of one copy with the lower half
// of the other, so each lane then holds both values (no LDS round trip).
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A operand from tile rows: row r, k-step ks (columns 16 ks + 8 hf .. + 7).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const uint4* s, int r, int ks, int hf) {
  return u4_bf8(s[upos<D>(r, 2 * ks + hf)]);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ i16x4 tr_read(const uint4* s, int row, int col) {
  const bf16* base = reinterpret_cast<const bf16*>(s);
  const int off = upos<D>(row, col >> 3) * 8 + (col & 7);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + off));
}
// A operand from tile columns: lane l gets column 32 dt + (l & 31) at rows
// 16 ks + 4 hf + 0..3 (slots 0..3) and 16 ks + 8 + 4 hf + 0..3 (slots 4..7).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint4* s, int dt, int ks, int lane) {
  const int i = lane & 15, g = lane >> 4, hf = lane >> 5;
  const int col = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
  const int row = 16 * ks + 4 * hf + (i >> 2);
  const i16x4 a = tr_read<D>(s, row, col);
  const i16x4 b = tr_read<D>(s, row + 8, col);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------------ forward (MFMA)
// Launch order of the causal MFMA kernels: a 1-D grid of (row blocks x H x B)
// workgroups whose ids are dealt heaviest row block first across every
// (batch, head) pair, so the lightest blocks form the tail of the launch.
// With H * B a multiple of 8, all blocks of one (batch, head) land on the
// same XCD (ids are dealt round-robin to the 8 XCDs) and share K/V in its L2.
// rank 0 is the heaviest: the last query block (forward, dQ) or the first
// key block (dK/dV).
__device__ __forceinline__ void attn_block(int T, int H, int& rank, int& h, int& b) {
  const int HB = gridDim.x / ((T + 127) / 128);
  const int id = blockIdx.x;
  rank = id / HB;
  const int bh = id - rank * HB;
  h = bh % H;
  b = bh / H;
}
// FIXED: the scores are known to lie below shift_log2 (in log2 units), so
// every exponent uses that constant shift instead of a running maximum:
// softmax is shift-invariant, and with QK-norm |q . k| <= |q| |k| <= D bounds
// the scaled score by sqrt(D), so exp2 neither overflows nor underflows.
// side / nattn: blocks nattn.. of the grid run the transpose jobs `side`
// instead (work that does not depend on the attention): dispatched after
// every attention block, they fill the CUs that the short query blocks free
// while the long ones finish.
template <int D, bool FIXED>
__global__ __launch_bounds__(256, 2) void attn_fwd_mfma(int T, int H, const bf16* __restrict__ qkv,
                                                        bf16* __restrict__ o, float* __restrict__ lse,
                                                        float scale_log2, float shift_log2, int W,
                                                        const TransposeJobs side, int nattn) {
  constexpr int KS = D / 16, DT = D / 32, KU = D / 8;
  __shared__ uint4 sK[2][64 * KU];
  __shared__ uint4 sV[2][64 * KU];
  if ((int)blockIdx.x >= nattn) {
    transpose_block(side, blockIdx.x - nattn);
    return;
  }
  const int nqb = (T + 127) / 128;
  const int HB = nattn / nqb;
  const int rank = blockIdx.x / HB, bh = blockIdx.x - rank * HB;
  const int h = bh % H, b = bh / H;
  const int qb = nqb - 1 - rank;
  const int C = H * D;
  const long ld = 3L * C;
  const bf16* Qg = qkv + (long)b * T * ld + h * D;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hf = lane >> 5;
  const int q0 = qb * 128;
  const int qw = q0 + 32 * wave;
  const int qi = qw + li;

  const __amdgpu_buffer_rsrc_t rQ = slice_rsrc(Qg, T, ld, D);
  const __amdgpu_buffer_rsrc_t rK = slice_rsrc(Kg, T, ld, D);
  const __amdgpu_buffer_rsrc_t rV = slice_rsrc(Vg, T, ld, D);
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = u4_bf8(bload(rQ, qi < T ? (uint32_t)(((long)qi * ld + 16 * s + 8 * hf) * 2) : OOB));

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
  float m_run = FIXED ? shift_log2 : -INFINITY, l_run = 0.0f;

  const int kv_end = min(T, q0 + 128);
  const int ntiles = (kv_end + 63) / 64;
  // with a window of W keys, query i sees keys i - W + 1 .. i: the block's
  // first tile is the one holding key q0 - W + 1
  const int t_first = W > 0 ? max(0, q0 - W + 1) / 64 : 0;
  RowTile<D>::direct(sK[0], rK, ld, 64 * t_first, T);
  RowTile<D>::direct(sV[0], rV, ld, 64 * t_first, T);
  wait_lds_loads();
  __syncthreads();

  // the loop is unrolled by two so that every LDS buffer index is a
  // compile-time constant: the compiler can then tell the next tile's
  // asynchronous copies from this tile's reads and inserts no wait between
  auto tile = [&](int t, auto curc) {
    constexpr int cur = decltype(curc)::value;
    const bool more = t + 1 < ntiles;
    const int kv0 = t * 64;
    if (more) {
      RowTile<D>::direct(sK[cur ^ 1], rK, ld, kv0 + 64, T);
      RowTile<D>::direct(sV[cur ^ 1], rV, ld, kv0 + 64, T);
    }
    if (kv0 <= qw + 31 && qw < T && (W == 0 || kv0 + 63 > qw - W)) {
      // S^T = K Q^T for two 32-key sub-tiles; k-step s+1 fragments are read
      // while the MFMAs of step s run
      f32x16 st[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[jt][r] = 0.0f;
      bf16x8 kfr[2][2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) kfr[0][jt] = row_frag<D>(sK[cur], 32 * jt + li, 0, hf);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) kfr[(s + 1) & 1][jt] = row_frag<D>(sK[cur], 32 * jt + li, s + 1, hf);
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          st[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[s & 1][jt], qf[s], st[jt], 0, 0, 0);
      }
      // online softmax in the log2 domain; the causal mask is applied only on
      // tiles that cross the diagonal or the sequence end (uniform branch)
      // raw scores; the log2-domain scale is folded into the exponent's FMA
      float p[2][16];
      auto scores = [&](auto masked) {
        float mx = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = st[jt][r];
            if constexpr (decltype(masked)::value) {
              const int j = kv0 + 32 * jt + 8 * (r >> 2) + 4 * hf + (r & 3);
              if (j > qi || j >= T || (W > 0 && j <= qi - W)) x = -INFINITY;
            }
            p[jt][r] = x;
            mx = fmaxf(mx, x);
          }
        return mx;
      };
      const bool need_mask = (kv0 + 63 > qw) || (kv0 + 64 > T) || (W > 0 && kv0 <= qw + 31 - W);
      float mx = need_mask ? scores(std::true_type{}) : scores(std::false_type{});
      float m_new = m_run, msub = m_run;
      bool dead = false;
      if constexpr (!FIXED) {
        mx = pair32_max(mx);
        m_new = fmaxf(m_run, mx * scale_log2);
        dead = (m_new == -INFINITY);
        msub = dead ? 0.0f : m_new;
      }
      float rs = 0.0f;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(p[jt][r], scale_log2, -msub));
          p[jt][r] = e;
          rs += e;
        }
      rs = pair32_sum(rs);
      // rescale the running sums only when some row's maximum grew (a
      // factor of exactly 1 otherwise)
      if constexpr (!FIXED) {
        if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
          const float corr = dead ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= corr;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= corr;
        }
      }
      l_run += rs;
      m_run = m_new;
      // O^T += V^T P^T; V^T fragments of step ks+1 are read during step ks
      bf16x8 vfr[2][DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vfr[0][dt] = tr_frag<D>(sV[cur], dt, 0, lane);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks + 1 < 4) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) vfr[(ks + 1) & 1][dt] = tr_frag<D>(sV[cur], dt, ks + 1, lane);
        }
        const bf16x8 pb = pack_slots(p[ks >> 1], 2 * (ks & 1));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[ks & 1][dt], pb, acc[dt], 0, 0, 0);
      }
    }
    wait_lds_loads();
    __syncthreads();
  };
  for (int t = t_first; t < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
  }

  if (qi < T) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    bf16* orow = o + ((long)b * T + qi) * C + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        uint2 u;
        u.x = pack2(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv);
        u.y = pack2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = u;
      }
    if (hf == 0) lse[((long)b * H + h) * T + qi] = (m_run + log2f(l_run)) * LN2;
  }
}

// QK-norm and RoPE backward applied to one row of a q or k gradient held as
// MFMA accumulators g[dt][r] (column d = 32 dt + 8 (r / 4) + 4 hf + r % 4;
// the two lane halves hold the two halves of the row).  y is the forward
// output (normalised, rotated) row, r_inv its saved 1 / rms, t its position.
// QK-norm: g <- r_inv (g - y mean(g * y)); RoPE: rotate pairs (i, i + D/2)
// by -t theta_i.
template <int D>
__device__ __forceinline__ void qk_row_bwd(float (&g)[D / 32][16], const bf16* __restrict__ yrow, float r_inv,
                                           const float2* __restrict__ cs_row, int hf, int rope, int qk_norm) {
  constexpr int DT = D / 32;
  if (qk_norm) {
    float y[DT][16];
    float part = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 u = *reinterpret_cast<const uint2*>(yrow + 32 * dt + 8 * q + 4 * hf);
        y[dt][4 * q + 0] = __uint_as_float(u.x << 16);
        y[dt][4 * q + 1] = __uint_as_float(u.x & 0xffff0000u);
        y[dt][4 * q + 2] = __uint_as_float(u.y << 16);
        y[dt][4 * q + 3] = __uint_as_float(u.y & 0xffff0000u);
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(g[dt][4 * q + e], y[dt][4 * q + e], part);
      }
    part = pair32_sum(part);
    const float m = part / D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) g[dt][r] = r_inv * (g[dt][r] - y[dt][r] * m);
  }
  if (rope) {
#pragma unroll
    for (int dt = 0; dt < DT / 2; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 32 * dt + 8 * q + 4 * hf;
        const float4 c01 = *reinterpret_cast<const float4*>(cs_row + i);
        const float4 c23 = *reinterpret_cast<const float4*>(cs_row + i + 2);
        const float cc[4] = {c01.x, c01.z, c23.x, c23.z}, ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = g[dt][4 * q + e], b2 = g[dt + DT / 2][4 * q + e];
          g[dt][4 * q + e] = a * cc[e] + b2 * ss[e];
          g[dt + DT / 2][4 * q + e] = b2 * cc[e] - a * ss[e];
        }
      }
  }
}

// ------------------------------------------------------ backward dK, dV (MFMA)
// A workgroup owns 128 keys of one (batch, head) and runs 8 waves as 4
// pairs; a pair owns 32 keys (one lane per key and lane half) and splits the
// work of every 32-query half tile n:
//   wave a (waves 0-3): S(n) = Q K^T, then P(n) = exp(S - lse) and
//       dS(n) = P (dP - delta), then dV^T += dO^T P;
//   wave b (waves 4-7): dP(n) = dO V^T, then dK^T += Q^T dS.
// dP goes b -> a and dS goes a -> b through LDS.  b runs one half ahead on
// dP and a one half ahead on S, so the two waves of a pair (which share a
// SIMD) alternate: while a works through the exponentials, b's MFMAs run.
// Each wave holds one 32-key accumulator set (dV or dK) and one set of key
// fragments (K or V), so two waves fit per SIMD.  Periods, separated by
// workgroup barriers (n = 2t + it for query tile t):
//   A(n): a: P, dS of half n, dV += ...;   b: dP(n + 1)
//   B(n): a: S(n + 1);                     b: dK += dS(n) ...
// Query tiles (Q, dO, log-sum-exp, delta) stream global -> LDS through three
// buffers: tile t + 2 is issued at A(2t) into the buffer of tile t - 1, and
// tile t + 1 must have landed before A(2t + 1).  The tile loop is unrolled by
// three so that every buffer index is a compile-time constant (the compiler
// then inserts no wait behind the copies in flight).
template <int D>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_mfma(int T, int H, const bf16* __restrict__ qkv,
                                                             const bf16* __restrict__ dO,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ delta,
                                                             bf16* __restrict__ dqkv, float scale_log2,
                                                             float scale, QkBwd qk, int W) {
  constexpr int KS = D / 16, DT = D / 32, KU = D / 8;
  constexpr int NCP = 2 * (64 * KU / 512);  // tile copies per wave (Q and dO)
  __shared__ uint4 sQ[3][64 * KU];
  __shared__ uint4 sdO[3][64 * KU];
  // log-sum-exp and delta per buffer as separate arrays (each a distinct
  // object to the compiler's alias analysis)
  __shared__ float sL0[64], sL1[64], sL2[64], sD0[64], sD1[64], sD2[64];
  __shared__ float4 xdP[4][2][4][64];  // [pair][half parity][register quad][lane]
  __shared__ uint4 xdS[4][2][2][64];   // [pair][half parity][16-key step][lane]
  auto sLb = [&](auto bc) __attribute__((always_inline)) -> float* {
    constexpr int bf = decltype(bc)::value;
    return bf == 0 ? sL0 : bf == 1 ? sL1 : sL2;
  };
  auto sDb = [&](auto bc) __attribute__((always_inline)) -> float* {
    constexpr int bf = decltype(bc)::value;
    return bf == 0 ? sD0 : bf == 1 ? sD1 : sD2;
  };
  int rank, h, b;
  attn_block(T, H, rank, h, b);
  const int C = H * D;
  const long ld = 3L * C;
  const bf16* Qg = qkv + (long)b * T * ld + h * D;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const bf16* dOg = dO + (long)b * T * C + h * D;
  const float* Lg = lse + ((long)b * H + h) * T;
  const float* Dg = delta + ((long)b * H + h) * T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pair = wave & 3;
  const bool is_b = wave >= 4;
  const int li = lane & 31, hf = lane >> 5;
  const int k0 = rank * 128;
  const int kw = k0 + 32 * pair;
  const int kj = kw + li;

  const __amdgpu_buffer_rsrc_t rQ = slice_rsrc(Qg, T, ld, D);
  const __amdgpu_buffer_rsrc_t rO = slice_rsrc(dOg, T, C, D);
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(Lg, (long)T * 4);
  const __amdgpu_buffer_rsrc_t rD = make_rsrc(Dg, (long)T * 4);
  // the pair's key row fragments: K for wave a (S), V for wave b (dP)
  bf16x8 kv[KS];
  {
    const __amdgpu_buffer_rsrc_t rKV = slice_rsrc(is_b ? Vg : Kg, T, ld, D);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kv[s] = u4_bf8(bload(rKV, kj < T ? (uint32_t)(((long)kj * ld + 16 * s + 8 * hf) * 2) : OOB));
  }
  f32x16 acc[DT];  // dV^T (wave a) or dK^T (wave b) of the pair's keys
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

  const int t_begin = k0 / 64;
  // with a window of W keys the last query that sees key k0 + 127 is
  // k0 + 126 + W
  const int t_end = W > 0 ? (min(T - 1, k0 + 126 + W) / 64) + 1 : (T + 63) / 64;
  // Q and dO tiles by all 8 waves; every wave also copies the tile's 64
  // log-sum-exp and delta values (4 bytes a lane, the same bytes to the same
  // place), so that all waves issue the same number of copies and the wait
  // below needs no branch; rows at or past T read as zeros
  auto stage_issue = [&](int t, auto bc) __attribute__((always_inline)) {
    constexpr int bf = decltype(bc)::value;
    const int qt0 = t * 64;
    RowTile<D>::template direct_by<8>(sQ[bf], rQ, ld, qt0, T);
    RowTile<D>::template direct_by<8>(sdO[bf], rO, C, qt0, T);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (__attribute__((address_space(3))) void*)sLb(bc), 4,
                                             (uint32_t)((qt0 + lane) * 4), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (__attribute__((address_space(3))) void*)sDb(bc), 4,
                                             (uint32_t)((qt0 + lane) * 4), 0, 0, 0);
  };
  // every copy but the most recent tile's has landed
  auto wait_but_tile = [&]() __attribute__((always_inline)) { wait_loads_but<NCP + 2>(); };

  f32x16 S;  // wave a: scores of the next half, carried from B(n - 1) to A(n)
  // S or dP of half it of the tile in buffer bf (rows of Q or dO times the
  // pair's K or V fragments)
  auto scores = [&](f32x16& out, const uint4* src, int it) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) out[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(src, 32 * it + li, s, hf), kv[s], out, 0, 0, 0);
  };
  auto phase_dP = [&](auto bc, int it, int xb) __attribute__((always_inline)) {
    constexpr int bf = decltype(bc)::value;
    f32x16 dP;
    scores(dP, sdO[bf], it);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xdP[pair][xb][q][lane] = make_float4(dP[4 * q], dP[4 * q + 1], dP[4 * q + 2], dP[4 * q + 3]);
  };
  // wave a: P and dS of half it (tile t, buffer bf), dS to the partner, then
  // dV^T += dO^T P
  auto phase_P = [&](auto bc, int t, int it) __attribute__((always_inline)) {
    constexpr int bf = decltype(bc)::value;
    const int q0h = t * 64 + 32 * it;
    uint32_t pw[8], dw[8];
    auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int il = 32 * it + 8 * g + 4 * hf;
        const float4 L4 = *reinterpret_cast<const float4*>(sLb(bc) + il);
        const float4 D4 = *reinterpret_cast<const float4*>(sDb(bc) + il);
        const float4 P4 = xdP[pair][it][g][lane];
        const float Ls[4] = {L4.x * LOG2E, L4.y * LOG2E, L4.z * LOG2E, L4.w * LOG2E};
        const float Ds[4] = {D4.x, D4.y, D4.z, D4.w};
        const float dPs[4] = {P4.x, P4.y, P4.z, P4.w};
        float pv[4], dv4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = __builtin_amdgcn_exp2f(fmaf(S[4 * g + e], scale_log2, -Ls[e]));
          if constexpr (decltype(masked)::value) {
            const int qi = q0h + 8 * g + 4 * hf + e;
            if (qi < kj || qi >= T || kj >= T || (W > 0 && qi - W >= kj)) x = 0.0f;
          }
          pv[e] = x;
          dv4[e] = x * (dPs[e] - Ds[e]);
        }
        pw[2 * g] = pack2(pv[0], pv[1]);
        pw[2 * g + 1] = pack2(pv[2], pv[3]);
        dw[2 * g] = pack2(dv4[0], dv4[1]);
        dw[2 * g + 1] = pack2(dv4[2], dv4[3]);
      }
    };
    if ((q0h < kw + 31) || (q0h + 32 > T) || (kw + 32 > T) || (W > 0 && q0h + 31 - W >= kw)) probs(std::true_type{});
    else probs(std::false_type{});
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      xdS[pair][it][kh][lane] = make_uint4(dw[4 * kh], dw[4 * kh + 1], dw[4 * kh + 2], dw[4 * kh + 3]);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8 pb = u4_bf8(make_uint4(pw[4 * kh], pw[4 * kh + 1], pw[4 * kh + 2], pw[4 * kh + 3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(sdO[bf], dt, 2 * it + kh, lane), pb, acc[dt],
                                                          0, 0, 0);
    }
  };
  // wave b: dK^T += Q^T dS for half it (dS from the partner)
  auto phase_dK = [&](auto bc, int it) __attribute__((always_inline)) {
    constexpr int bf = decltype(bc)::value;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8 db = u4_bf8(xdS[pair][it][kh][lane]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(sQ[bf], dt, 2 * it + kh, lane), db, acc[dt],
                                                          0, 0, 0);
    }
  };

  // tile t in buffer c (= (t - t_begin) % 3); tile t + 1 in c1, t + 2 in c2.
  // Nothing inside depends on whether tiles t + 1, t + 2 exist: copies past
  // the last tile read as zeros, and the work on them (S, dP of a half past
  // the end) is dropped, so the waits the compiler derives need no merging
  // of paths.
  auto tile = [&](int t, auto cc) __attribute__((always_inline)) {
    constexpr int c = decltype(cc)::value;
    constexpr int c1 = (c + 1) % 3, c2 = (c + 2) % 3;
    using C0 = std::integral_constant<int, c>;
    using C1 = std::integral_constant<int, c1>;
    using C2 = std::integral_constant<int, c2>;
    // A(2t)
    stage_issue(t + 2, C2{});
    if (!is_b) phase_P(C0{}, t, 0);
    else phase_dP(C0{}, 1, 1);
    lds_barrier();
    // B(2t)
    if (!is_b) scores(S, sQ[c], 1);
    else phase_dK(C0{}, 0);
    wait_but_tile();
    lds_barrier();  // tile t + 1 has landed
    // A(2t + 1)
    if (!is_b) phase_P(C0{}, t, 1);
    else phase_dP(C1{}, 0, 0);
    lds_barrier();
    // B(2t + 1)
    if (!is_b) scores(S, sQ[c1], 0);
    else phase_dK(C0{}, 1);
    lds_barrier();
  };

  stage_issue(t_begin, std::integral_constant<int, 0>{});
  stage_issue(t_begin + 1, std::integral_constant<int, 1>{});
  wait_but_tile();
  lds_barrier();
  // before A(0): b forms dP(0), a forms S(0)
  if (is_b) phase_dP(std::integral_constant<int, 0>{}, 0, 0);
  else scores(S, sQ[0], 0);
  lds_barrier();
  for (int t = t_begin; t < t_end; t += 3) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_end) tile(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < t_end) tile(t + 2, std::integral_constant<int, 2>{});
  }
  wait_lds_loads();  // the copies issued past the last tile

  if (kj < T) {
    if (!is_b) {
      bf16* vrow = dqkv + ((long)b * T + kj) * ld + 2 * C + h * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * hf;
          uint2 u;
          u.x = pack2(acc[dt][4 * g], acc[dt][4 * g + 1]);
          u.y = pack2(acc[dt][4 * g + 2], acc[dt][4 * g + 3]);
          *reinterpret_cast<uint2*>(vrow + d) = u;
        }
    } else {
      bf16* krow = dqkv + ((long)b * T + kj) * ld + C + h * D;
      float gk[DT][16];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) gk[dt][r] = acc[dt][r] * scale;
      if (qk.rope | qk.qk_norm) {
        const long n = (long)b * T + kj;
        const float r_inv = qk.qk_norm ? qk.rstd[(long)qk.N * H + n * H + h] : 1.0f;
        qk_row_bwd<D>(gk, Kg + (long)kj * ld, r_inv, qk.rope ? qk.cs + (long)kj * (D / 2) : nullptr, hf, qk.rope,
                       qk.qk_norm);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * hf;
          uint2 u;
          u.x = pack2(gk[dt][4 * g], gk[dt][4 * g + 1]);
          u.y = pack2(gk[dt][4 * g + 2], gk[dt][4 * g + 3]);
          *reinterpret_cast<uint2*>(krow + d) = u;
        }
    }
  }
}

// ---------------------------------------------------------- backward dQ (MFMA)
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_mfma(int T, int H, const bf16* __restrict__ qkv,
                                                           const bf16* __restrict__ o,
                                                           const bf16* __restrict__ dO,
                                                           const float* __restrict__ lse,
                                                           float* __restrict__ delta,
                                                           bf16* __restrict__ dqkv, float scale_log2,
                                                           float scale, QkBwd qk, int W) {
  constexpr int KS = D / 16, DT = D / 32, KU = D / 8;
  __shared__ uint4 sK[2][64 * KU];
  __shared__ uint4 sV[2][64 * KU];
  const int nqb = (T + 127) / 128;
  int rank, h, b;
  attn_block(T, H, rank, h, b);
  const int qb = nqb - 1 - rank;
  const int C = H * D;
  const long ld = 3L * C;
  const bf16* Qg = qkv + (long)b * T * ld + h * D;
  const bf16* Kg = Qg + C;
  const bf16* Vg = Qg + 2 * C;
  const bf16* dOg = dO + (long)b * T * C + h * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, hf = lane >> 5;
  const int q0 = qb * 128;
  const int qw = q0 + 32 * wave;
  const int qi = qw + li;

  const __amdgpu_buffer_rsrc_t rQ = slice_rsrc(Qg, T, ld, D);
  const __amdgpu_buffer_rsrc_t rK = slice_rsrc(Kg, T, ld, D);
  const __amdgpu_buffer_rsrc_t rV = slice_rsrc(Vg, T, ld, D);
  const __amdgpu_buffer_rsrc_t rO = slice_rsrc(dOg, T, C, D);
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = u4_bf8(bload(rQ, qi < T ? (uint32_t)(((long)qi * ld + 16 * s + 8 * hf) * 2) : OOB));
    df[s] = u4_bf8(bload(rO, qi < T ? (uint32_t)(((long)qi * C + 16 * s + 8 * hf) * 2) : OOB));
  }
  const long row_lse = ((long)b * H + h) * T + qi;
  const float L2 = qi < T ? lse[row_lse] * LOG2E : 0.0f;
  // delta = rowsum(dO * O) of this query from the same row slices df holds;
  // the dK/dV pass, which runs next, reads it back
  float Dl;
  {
    const __amdgpu_buffer_rsrc_t rOo = slice_rsrc(o + (long)b * T * C + h * D, T, C, D);
    float part = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const bf16x8 ov = u4_bf8(bload(rOo, qi < T ? (uint32_t)(((long)qi * C + 16 * s2 + 8 * hf) * 2) : OOB));
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)ov[e], (float)df[s2][e], part);
    }
    Dl = pair32_sum(part);
    if (qi < T && hf == 0) delta[row_lse] = Dl;
  }
  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.0f;

  const int kv_end = min(T, q0 + 128);
  const int ntiles = (kv_end + 63) / 64;
  const int t_first = W > 0 ? max(0, q0 - W + 1) / 64 : 0;  // as in the forward
  RowTile<D>::direct(sK[0], rK, ld, 64 * t_first, T);
  RowTile<D>::direct(sV[0], rV, ld, 64 * t_first, T);
  wait_lds_loads();
  __syncthreads();
  // the loop is unrolled by two so that every LDS buffer index is a
  // compile-time constant: the compiler can then tell the next tile's
  // asynchronous copies from this tile's reads and inserts no wait between
  auto tile = [&](int t, auto curc) {
    constexpr int cur = decltype(curc)::value;
    const bool more = t + 1 < ntiles;
    const int kv0 = t * 64;
    if (more) {
      RowTile<D>::direct(sK[cur ^ 1], rK, ld, kv0 + 64, T);
      RowTile<D>::direct(sV[cur ^ 1], rV, ld, kv0 + 64, T);
    }
    if (kv0 <= qw + 31 && qw < T && (W == 0 || kv0 + 63 > qw - W)) {
      // the 64-key tile is processed as two 32-key halves: S^T = K Q^T and
      // dP^T = V dO^T for the half, dS^T, then dQ^T += K^T dS^T over it;
      // only one half's scores are live at a time
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        if (kv0 + 32 * jt > qw + 31) break;                        // half above the diagonal
        if (W > 0 && kv0 + 32 * jt + 31 <= qw - W) continue;       // half left of the window
        f32x16 St, dPt;
#pragma unroll
        for (int r = 0; r < 16; ++r) { St[r] = 0.0f; dPt[r] = 0.0f; }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          St = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(sK[cur], 32 * jt + li, s, hf), qf[s], St, 0, 0, 0);
          dPt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(sV[cur], 32 * jt + li, s, hf), df[s], dPt, 0, 0,
                                                        0);
        }
        float ds[16];
        auto grads = [&](auto masked) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float pv = __builtin_amdgcn_exp2f(fmaf(St[r], scale_log2, -L2));
            if constexpr (decltype(masked)::value) {
              const int j = kv0 + 32 * jt + 8 * (r >> 2) + 4 * hf + (r & 3);
              if (j > qi || j >= T || qi >= T || (W > 0 && j <= qi - W)) pv = 0.0f;
            }
            ds[r] = pv * (dPt[r] - Dl);
          }
        };
        const int k0 = kv0 + 32 * jt;
        if ((k0 + 31 > qw) || (k0 + 32 > T) || (qw + 32 > T) || (W > 0 && k0 <= qw + 31 - W))
          grads(std::true_type{});
        else grads(std::false_type{});
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const bf16x8 db = pack_slots(ds, 2 * kh);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(sK[cur], dt, 2 * jt + kh, lane), db, dq[dt],
                                                             0, 0, 0);
        }
      }
    }
    wait_lds_loads();
    __syncthreads();
  };
  for (int t = t_first; t < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
  }
  if (qi < T) {
    bf16* qrow = dqkv + ((long)b * T + qi) * ld + h * D;
    float gq[DT][16];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) gq[dt][r] = dq[dt][r] * scale;
    if (qk.rope | qk.qk_norm) {
      const long n = (long)b * T + qi;
      const float r_inv = qk.qk_norm ? qk.rstd[n * H + h] : 1.0f;
      qk_row_bwd<D>(gq, Qg + (long)qi * ld, r_inv, qk.rope ? qk.cs + (long)qi * (D / 2) : nullptr, hf, qk.rope,
                     qk.qk_norm);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        uint2 u;
        u.x = pack2(gq[dt][4 * g], gq[dt][4 * g + 1]);
        u.y = pack2(gq[dt][4 * g + 2], gq[dt][4 * g + 3]);
        *reinterpret_cast<uint2*>(qrow + d) = u;
      }
  }
}

// ------------------------------------------------------------ SIMT fallbacks
// One thread per query (forward, dQ) or per key (dK, dV); fp32 arithmetic.
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_fwd_simt(int TT, int H, const T* __restrict__ qkv, T* __restrict__ o,
                                                    float* __restrict__ lse, float scale, int W) {
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (qi >= TT) return;
  const int C = H * D;
  const long ld = 3L * C;
  const T* base = qkv + (long)b * TT * ld + h * D;
  float q[D], acc[D];
  for (int d = 0; d < D; ++d) { q[d] = to_f32(base[(long)qi * ld + d]) * scale; acc[d] = 0.0f; }
  float m = -INFINITY, l = 0.0f;
  for (int j = W > 0 ? max(0, qi - W + 1) : 0; j <= qi; ++j) {
    const T* kr = base + (long)j * ld + C;
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = fmaf(q[d], to_f32(kr[d]), s);
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);
    const float pj = expf(s - mn);
    l = l * corr + pj;
    const T* vr = kr + C;
    for (int d = 0; d < D; ++d) acc[d] = fmaf(pj, to_f32(vr[d]), acc[d] * corr);
    m = mn;
  }
  T* orow = o + ((long)b * TT + qi) * C + h * D;
  for (int d = 0; d < D; ++d) orow[d] = from_f32<T>(acc[d] / l);
  lse[((long)b * H + h) * TT + qi] = m + logf(l);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_simt(int TT, int H, const T* __restrict__ qkv,
                                                       const T* __restrict__ dO, const float* __restrict__ lse,
                                                       const float* __restrict__ delta, T* __restrict__ dqkv,
                                                       float scale, int W) {
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (qi >= TT) return;
  const int C = H * D;
  const long ld = 3L * C;
  const T* base = qkv + (long)b * TT * ld + h * D;
  const T* dob = dO + ((long)b * TT + qi) * C + h * D;
  float q[D], g[D], acc[D];
  for (int d = 0; d < D; ++d) { q[d] = to_f32(base[(long)qi * ld + d]); g[d] = to_f32(dob[d]); acc[d] = 0.0f; }
  const long rl = ((long)b * H + h) * TT + qi;
  const float L = lse[rl], Dl = delta[rl];
  for (int j = W > 0 ? max(0, qi - W + 1) : 0; j <= qi; ++j) {
    const T* kr = base + (long)j * ld + C;
    const T* vr = kr + C;
    float s = 0.0f, dp = 0.0f;
    for (int d = 0; d < D; ++d) { s = fmaf(q[d], to_f32(kr[d]), s); dp = fmaf(g[d], to_f32(vr[d]), dp); }
    const float p = expf(s * scale - L);
    const float ds = p * (dp - Dl);
    for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, to_f32(kr[d]), acc[d]);
  }
  T* out = dqkv + ((long)b * TT + qi) * ld + h * D;
  for (int d = 0; d < D; ++d) out[d] = from_f32<T>(acc[d] * scale);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_simt(int TT, int H, const T* __restrict__ qkv,
                                                         const T* __restrict__ dO, const float* __restrict__ lse,
                                                         const float* __restrict__ delta, T* __restrict__ dqkv,
                                                         float scale, int W) {
  const int kj = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (kj >= TT) return;
  const int C = H * D;
  const long ld = 3L * C;
  const T* base = qkv + (long)b * TT * ld + h * D;
  float k[D], v[D], dk[D], dv[D];
  for (int d = 0; d < D; ++d) {
    k[d] = to_f32(base[(long)kj * ld + C + d]);
    v[d] = to_f32(base[(long)kj * ld + 2 * C + d]);
    dk[d] = 0.0f; dv[d] = 0.0f;
  }
  const int i_end = W > 0 ? min(TT, kj + W) : TT;
  for (int i = kj; i < i_end; ++i) {
    const T* qr = base + (long)i * ld;
    const T* gr = dO + ((long)b * TT + i) * C + h * D;
    const long rl = ((long)b * H + h) * TT + i;
    float s = 0.0f, dp = 0.0f;
    for (int d = 0; d < D; ++d) { s = fmaf(to_f32(qr[d]), k[d], s); dp = fmaf(to_f32(gr[d]), v[d], dp); }
    const float p = expf(s * scale - lse[rl]);
    const float ds = p * (dp - delta[rl]);
    for (int d = 0; d < D; ++d) { dk[d] = fmaf(ds, to_f32(qr[d]), dk[d]); dv[d] = fmaf(p, to_f32(gr[d]), dv[d]); }
  }
  T* out = dqkv + ((long)b * TT + kj) * ld + C + h * D;
  for (int d = 0; d < D; ++d) { out[d] = from_f32<T>(dk[d] * scale); out[C + d] = from_f32<T>(dv[d]); }
}

// ----------------------------------------------------- RoPE / QK-norm, delta
// (the RoPE table itself is written by the norm1 launch: rope_entry)
// One wavefront per (row, head, q|k); lane i < D/2 handles pair (i, i + D/2).
template <typename T>
__global__ __launch_bounds__(256) void qk_fwd_k(int N, int TT, int H, int D, int rope, int qk_norm, float eps,
                                                const float2* __restrict__ cs, T* __restrict__ qkv,
                                                float* __restrict__ rstd) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= 2L * N * H) return;
  const int which = (int)(w / ((long)N * H));
  const long rem = w % ((long)N * H);
  const int n = (int)(rem / H), h = (int)(rem % H);
  const int C = H * D, half = D / 2;
  const int t = n % TT;
  T* v = qkv + (long)n * 3 * C + which * C + h * D;
  // D <= 128: one pass of 64 lanes covers every pair
  const int i = lane;
  float a = 0.0f, bb = 0.0f;
  if (i < half) { a = to_f32(v[i]); bb = to_f32(v[i + half]); }
  float r = 1.0f;
  if (qk_norm) {
    const float ss = wave_sum(a * a + bb * bb);
    r = 1.0f / sqrtf(ss / D + eps);
  }
  if (i < half) {
    float na = a, nb = bb;
    if (rope) {
      const float2 c = cs[t * half + i];
      na = a * c.x - bb * c.y;
      nb = a * c.y + bb * c.x;
    }
    v[i] = from_f32<T>(na * r);
    v[i + half] = from_f32<T>(nb * r);
  }
  if (qk_norm && lane == 0) rstd[(long)which * N * H + (long)n * H + h] = r;
}

template <typename T>
__global__ __launch_bounds__(256) void qk_bwd_k(int N, int TT, int H, int D, int rope, int qk_norm,
                                                const float2* __restrict__ cs, const T* __restrict__ qkv,
                                                const float* __restrict__ rstd, T* __restrict__ dqkv) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= 2L * N * H) return;
  const int which = (int)(w / ((long)N * H));
  const long rem = w % ((long)N * H);
  const int n = (int)(rem / H), h = (int)(rem % H);
  const int C = H * D, half = D / 2;
  const int t = n % TT;
  const long off = (long)n * 3 * C + which * C + h * D;
  const int i = lane;
  float ga = 0.0f, gb = 0.0f, ya = 0.0f, yb = 0.0f;
  if (i < half) {
    ga = to_f32(dqkv[off + i]); gb = to_f32(dqkv[off + i + half]);
    ya = to_f32(qkv[off + i]); yb = to_f32(qkv[off + i + half]);
  }
  if (qk_norm) {
    const float r = rstd[(long)which * N * H + (long)n * H + h];
    const float m = wave_sum(ga * ya + gb * yb) / D;
    ga = r * (ga - ya * m);
    gb = r * (gb - yb * m);
  }
  if (i < half) {
    if (rope) {
      const float2 c = cs[t * half + i];
      const float na = ga * c.x + gb * c.y;
      const float nb = -ga * c.y + gb * c.x;
      ga = na; gb = nb;
    }
    dqkv[off + i] = from_f32<T>(ga);
    dqkv[off + i + half] = from_f32<T>(gb);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void delta_k(int N, int TT, int H, int D, const T* __restrict__ o,
                                               const T* __restrict__ dO, float* __restrict__ delta) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)N * H) return;
  const int n = (int)(idx / H), h = (int)(idx % H);
  const int C = H * D;
  const T* a = o + (long)n * C + h * D;
  const T* g = dO + (long)n * C + h * D;
  float s = 0.0f;
  for (int d = 0; d < D; d += 8) {
    float x[8], y[8];
    Vec8<T>::load(a + d, x);
    Vec8<T>::load(g + d, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(x[e], y[e], s);
  }
  const int b = n / TT, t = n % TT;
  delta[((long)b * H + h) * TT + t] = s;
}

template <typename T, int D>
hipError_t simt_all(int which, int B, int TT, int H, const void* qkv, const void* dO, void* out, float* lse,
                    const float* delta, int W, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)D);
  dim3 grid(cdiv(TT, 64), H, B);
  if (which == 0)
    hipLaunchKernelGGL((attn_fwd_simt<T, D>), grid, dim3(64), 0, s, TT, H, (const T*)qkv, (T*)out, lse, scale, W);
  else if (which == 1)
    hipLaunchKernelGGL((attn_bwd_dq_simt<T, D>), grid, dim3(64), 0, s, TT, H, (const T*)qkv, (const T*)dO, lse,
                       delta, (T*)out, scale, W);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_simt<T, D>), grid, dim3(64), 0, s, TT, H, (const T*)qkv, (const T*)dO, lse,
                       delta, (T*)out, scale, W);
  return hipGetLastError();
}

template <typename T>
hipError_t simt_dispatch(int which, int B, int TT, int H, int D, const void* qkv, const void* dO, void* out,
                         float* lse, const float* delta, int W, hipStream_t s) {
  switch (D) {
    case 16: return simt_all<T, 16>(which, B, TT, H, qkv, dO, out, lse, delta, W, s);
    case 32: return simt_all<T, 32>(which, B, TT, H, qkv, dO, out, lse, delta, W, s);
    case 64: return simt_all<T, 64>(which, B, TT, H, qkv, dO, out, lse, delta, W, s);
    case 128: return simt_all<T, 128>(which, B, TT, H, qkv, dO, out, lse, delta, W, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool attn_mfma_supported(int dtype, int D) { return dtype == 1 && (D == 64 || D == 128); }

hipError_t launch_qk_fwd(int dtype, int B, int T, int H, int D, int rope, int qk_norm, float eps,
                         const float2* cs, void* qkv, float* rstd, hipStream_t s) {
  const int N = B * T;
  const long waves = 2L * N * H;
  dim3 grid((unsigned)cdiv(waves, 4));
  if (dtype == 1)
    hipLaunchKernelGGL(qk_fwd_k<bf16>, grid, dim3(256), 0, s, N, T, H, D, rope, qk_norm, eps, cs, (bf16*)qkv, rstd);
  else
    hipLaunchKernelGGL(qk_fwd_k<float>, grid, dim3(256), 0, s, N, T, H, D, rope, qk_norm, eps, cs, (float*)qkv, rstd);
  return hipGetLastError();
}

hipError_t launch_qk_bwd(int dtype, int B, int T, int H, int D, int rope, int qk_norm, const float2* cs,
                         const void* qkv, const float* rstd, void* dqkv, hipStream_t s) {
  const int N = B * T;
  const long waves = 2L * N * H;
  dim3 grid((unsigned)cdiv(waves, 4));
  if (dtype == 1)
    hipLaunchKernelGGL(qk_bwd_k<bf16>, grid, dim3(256), 0, s, N, T, H, D, rope, qk_norm, cs, (const bf16*)qkv, rstd,
                       (bf16*)dqkv);
  else
    hipLaunchKernelGGL(qk_bwd_k<float>, grid, dim3(256), 0, s, N, T, H, D, rope, qk_norm, cs, (const float*)qkv,
                       rstd, (float*)dqkv);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(int dtype, int B, int T, int H, int D, int qk_norm, int window, const void* qkv,
                           void* o, float* lse, const TransposeDesc* side, int nside, hipStream_t s) {
  const int W = window >= T ? 0 : window;  // a window of T or more keys is the full causal mask
  if (attn_mfma_supported(dtype, D)) {
    const float scale_log2 = LOG2E / sqrtf((float)D);
    // with QK-norm |q|, |k| <= sqrt(D) (up to bf16 rounding), so a scaled
    // score is at most sqrt(D); the shift adds 3% for the rounding
    const float shift_log2 = 1.03f * sqrtf((float)D) * LOG2E;
    if (nside < 0 || nside > TRANSPOSE_MAX) return hipErrorInvalidValue;
    TransposeJobs J{};
    const int nj = nside ? make_transpose_jobs(side, nside, J) : 0;
    const int nattn = cdiv(T, 128) * H * B;
    dim3 grid(nattn + nj);
#define AF(DD, FX) hipLaunchKernelGGL((attn_fwd_mfma<DD, FX>), grid, dim3(256), 0, s, T, H, (const bf16*)qkv, \
                                      (bf16*)o, lse, scale_log2, shift_log2, W, J, nattn)
    if (D == 128) {
      if (qk_norm) AF(128, true); else AF(128, false);
    } else {
      if (qk_norm) AF(64, true); else AF(64, false);
    }
#undef AF
    return hipGetLastError();
  }
  hipError_t e = dtype == 1 ? simt_dispatch<bf16>(0, B, T, H, D, qkv, nullptr, o, lse, nullptr, W, s)
                            : simt_dispatch<float>(0, B, T, H, D, qkv, nullptr, o, lse, nullptr, W, s);
  if (e == hipSuccess && nside) e = launch_transpose(side, nside, s);
  return e;
}

hipError_t launch_attn_delta(int dtype, int B, int T, int H, int D, const void* o, const void* dO, float* delta,
                             hipStream_t s) {
  const int N = B * T;
  dim3 grid(cdiv((long)N * H, 256));
  if (dtype == 1)
    hipLaunchKernelGGL(delta_k<bf16>, grid, dim3(256), 0, s, N, T, H, D, (const bf16*)o, (const bf16*)dO, delta);
  else
    hipLaunchKernelGGL(delta_k<float>, grid, dim3(256), 0, s, N, T, H, D, (const float*)o, (const float*)dO, delta);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkdv(int dtype, int B, int T, int H, int D, int window, const void* qkv, const void* dO,
                                const float* lse, const float* delta, void* dqkv, const QkBwd& qk, hipStream_t s) {
  const int W = window >= T ? 0 : window;
  if (attn_mfma_supported(dtype, D)) {
    const float scale = 1.0f / sqrtf((float)D);
    const float scale_log2 = LOG2E * scale;
    dim3 g(cdiv(T, 128) * H * B);
    if (D == 128)
      hipLaunchKernelGGL(attn_bwd_dkdv_mfma<128>, g, dim3(512), 0, s, T, H, (const bf16*)qkv, (const bf16*)dO, lse,
                         delta, (bf16*)dqkv, scale_log2, scale, qk, W);
    else
      hipLaunchKernelGGL(attn_bwd_dkdv_mfma<64>, g, dim3(512), 0, s, T, H, (const bf16*)qkv, (const bf16*)dO, lse,
                         delta, (bf16*)dqkv, scale_log2, scale, qk, W);
    return hipGetLastError();
  }
  if (dtype == 1) return simt_dispatch<bf16>(2, B, T, H, D, qkv, dO, dqkv, (float*)lse, delta, W, s);
  return simt_dispatch<float>(2, B, T, H, D, qkv, dO, dqkv, (float*)lse, delta, W, s);
}

hipError_t launch_attn_bwd_dq(int dtype, int B, int T, int H, int D, int window, const void* qkv, const void* o,
                              const void* dO, const float* lse, float* delta, void* dqkv, const QkBwd& qk,
                              hipStream_t s) {
  const int W = window >= T ? 0 : window;
  if (attn_mfma_supported(dtype, D)) {
    const float scale = 1.0f / sqrtf((float)D);
    const float scale_log2 = LOG2E * scale;
    dim3 g(cdiv(T, 128) * H * B);
    if (D == 128)
      hipLaunchKernelGGL(attn_bwd_dq_mfma<128>, g, dim3(256), 0, s, T, H, (const bf16*)qkv, (const bf16*)o,
                         (const bf16*)dO, lse, delta, (bf16*)dqkv, scale_log2, scale, qk, W);
    else
      hipLaunchKernelGGL(attn_bwd_dq_mfma<64>, g, dim3(256), 0, s, T, H, (const bf16*)qkv, (const bf16*)o,
                         (const bf16*)dO, lse, delta, (bf16*)dqkv, scale_log2, scale, qk, W);
    return hipGetLastError();
  }
  if (dtype == 1) return simt_dispatch<bf16>(1, B, T, H, D, qkv, dO, dqkv, (float*)lse, delta, W, s);
  return simt_dispatch<float>(1, B, T, H, D, qkv, dO, dqkv, (float*)lse, delta, W, s);
}
