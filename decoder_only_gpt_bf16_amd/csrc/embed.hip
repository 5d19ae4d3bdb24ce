// Token (+ learned position) embedding forward and backward.
//
// Forward ("nanoGPT — Karpathy's minimal GPT pretraining repo", model.py:
// token embeddings wte plus learned absolute positions wpe): a gather, one
// wavefront per token row with 16-byte loads.
//
// Backward: dwte[v] = sum of dx0 rows whose id is v, in a fixed order, with
// no floating-point atomics.  The (id, position) pairs are sorted as 64-bit
// keys id << 32 | position (all distinct, so the order is by id, then by
// position) with a bitonic network: tiles of SORT_TILE keys sort in LDS, and
// merge stages with strides of a tile or more run as passes over global
// memory.  Ids are skewed (e.g. Zipf: a few ids own thousands of rows); the
// sorted list is cut into chunks of CHUNK entries, and one wave per chunk
// sums each run of equal ids in position order.  A run wholly inside a chunk
// is written directly; a run crossing chunk boundaries leaves its pieces in
// per-chunk slots that a second kernel adds in chunk order.
// dwpe[t] = sum over the batch of dx0[b, t].
#include "kernels.h"

namespace {

constexpr int CHUNK = 16;
constexpr int MAXV = 4;  // 8-wide vectors per lane: C <= 64 * 8 * 4

template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_k(int N, int TT, int C, int V, const int32_t* __restrict__ ids,
                                                   const T* __restrict__ wte, const T* __restrict__ wpe,
                                                   T* __restrict__ x0) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const int id = ids[n];
  const bool ok = id >= 0 && id < V;
  const int t = n % TT;
  for (int c = lane * 8; c < C; c += 64 * 8) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0}, p[8];
    if (ok) Vec8<T>::load(wte + (long)id * C + c, a);
    if (wpe) {
      Vec8<T>::load(wpe + (long)t * C + c, p);
      for (int e = 0; e < 8; ++e) a[e] += p[e];
    }
    Vec8<T>::store(x0 + (long)n * C + c, a);
  }
}

// Sort keys: (id, or V for an id outside [0, V), whose run is then skipped)
// << 32 | position, padded to P (a power of two) with all-ones keys that sort
// last.
__global__ void sort_keys_k(int N, int P, int V, const int32_t* __restrict__ ids, uint64_t* __restrict__ k) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  if (i < N) {
    const int id = ids[i];
    const uint32_t key = (id >= 0 && id < V) ? (uint32_t)id : (uint32_t)V;
    k[i] = ((uint64_t)key << 32) | (uint32_t)i;
  } else {
    k[i] = ~0ull;
  }
}

// Bitonic network, ascending over P = 2^p keys: in merge m (2, 4, .., P)
// the stage of stride s (m / 2, .., 1) orders each pair (i, i + s) with
// i & s == 0, ascending when i & m == 0 and descending otherwise.
constexpr int SORT_TILE = 8192;  // keys per LDS tile (64 KB)
constexpr int SORT_THREADS = 1024;

__device__ __forceinline__ void cmp_swap(uint64_t& a, uint64_t& b, bool up) {
  if ((a > b) == up) {
    const uint64_t t = a;
    a = b;
    b = t;
  }
}

// One block per tile of n = min(P, SORT_TILE) keys: the merges m_lo .. m_hi
// (powers of two), each from stride min(m / 2, n / 2) down to 1, in LDS.
// The initial sort takes m_lo = 2, m_hi = n; a merge m > n takes
// m_lo = m_hi = m after its global stages.
__global__ __launch_bounds__(SORT_THREADS) void bitonic_tile_k(uint64_t* __restrict__ k, int n, int m_lo,
                                                               int m_hi) {
  __shared__ uint64_t t[SORT_TILE];
  const long base = (long)blockIdx.x * n;
  for (int i = threadIdx.x; i < n; i += SORT_THREADS) t[i] = k[base + i];
  __syncthreads();
  for (int m = m_lo; m <= m_hi; m <<= 1) {
    for (int s = min(m, n) >> 1; s > 0; s >>= 1) {
      for (int q = threadIdx.x; q < n / 2; q += SORT_THREADS) {
        const int i = (q / s) * 2 * s + (q % s);  // lower element of the pair
        const bool up = ((base + i) & m) == 0;
        cmp_swap(t[i], t[i + s], up);
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += SORT_THREADS) k[base + i] = t[i];
}

// One stage (merge m, stride s >= the tile size) over global memory: one
// thread per pair.
__global__ __launch_bounds__(256) void bitonic_pass_k(uint64_t* __restrict__ k, long P, long m, long s) {
  const long q = (long)blockIdx.x * 256 + threadIdx.x;
  if (q >= P / 2) return;
  const long i = (q / s) * 2 * s + (q % s);
  uint64_t a = k[i], b = k[i + s];
  cmp_swap(a, b, (i & m) == 0);
  k[i] = a;
  k[i + s] = b;
}

// Split the sorted keys into ids and positions (first N entries).
__global__ void split_keys_k(int N, const uint64_t* __restrict__ k, int32_t* __restrict__ skeys,
                             int32_t* __restrict__ spos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const uint64_t v = k[i];
  skeys[i] = (int32_t)(v >> 32);
  spos[i] = (int32_t)(v & 0xffffffffu);
}

__global__ void fill_i32_k(long n, int32_t* p, int32_t v) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = v;
}

// seg_start[v] / seg_end[v]: the run of id v in the sorted list (empty: -1).
__global__ void seg_bounds_k(int N, int V, const int32_t* __restrict__ skeys, int32_t* __restrict__ seg_start,
                             int32_t* __restrict__ seg_end) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const int v = skeys[i];
  if (v >= V) return;
  if (i == 0 || skeys[i - 1] != v) seg_start[v] = i;
  if (i == N - 1 || skeys[i + 1] != v) seg_end[v] = i + 1;
}

// One wave per chunk of CHUNK sorted entries.  slot[2*c] holds the piece of
// the run that enters chunk c from the left (or spans it), slot[2*c+1] the
// piece of the run that leaves it to the right.
template <typename T>
__global__ __launch_bounds__(256) void embed_chunk_k(int N, int C, int V, const int32_t* __restrict__ skeys,
                                                     const int32_t* __restrict__ spos, const T* __restrict__ dx0,
                                                     const int32_t* __restrict__ seg_start,
                                                     const int32_t* __restrict__ seg_end, float* __restrict__ dwte,
                                                     float* __restrict__ slots, int accumulate) {
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i0 = c * CHUNK;
  if (i0 >= N) return;
  const int i1 = min(N, i0 + CHUNK);
  int i = i0;
  while (i < i1) {
    const int v = skeys[i];
    if (v >= V) return;  // the out-of-range run sorts last
    const int rs = seg_start[v], re = seg_end[v];
    const int pe = min(re, i1);
    float acc[MAXV][8];
#pragma unroll
    for (int q = 0; q < MAXV; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] = 0.0f;
    for (int k = i; k < pe; ++k) {
      const T* row = dx0 + (long)spos[k] * C;
#pragma unroll
      for (int q = 0; q < MAXV; ++q) {
        const int col = (lane + 64 * q) * 8;
        if (col < C) {
          float x[8];
          Vec8<T>::load(row + col, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[q][e] += x[e];
        }
      }
    }
    float* dst;
    bool add = false;
    if (rs >= i0 && re <= i1) {           // whole run inside the chunk
      dst = dwte + (long)v * C;
      add = accumulate != 0;
    } else if (rs < i0) {                 // entered from the left (maybe spans)
      dst = slots + (long)(2 * c) * C;
    } else {                              // leaves to the right
      dst = slots + (long)(2 * c + 1) * C;
    }
#pragma unroll
    for (int q = 0; q < MAXV; ++q) {
      const int col = (lane + 64 * q) * 8;
      if (col < C) {
        float o[8];
        if (add) {
          Vec8<float>::load(dst + col, o);
          for (int e = 0; e < 8; ++e) o[e] += acc[q][e];
        } else {
          for (int e = 0; e < 8; ++e) o[e] = acc[q][e];
        }
        Vec8<float>::store(dst + col, o);
      }
    }
    i = pe;
  }
}

// One wave per vocabulary row: zero untouched rows (accumulate = 0) and
// assemble runs that cross chunk boundaries from their pieces, in order.
__global__ __launch_bounds__(256) void embed_rows_k(int V, int C, const int32_t* __restrict__ seg_start,
                                                    const int32_t* __restrict__ seg_end,
                                                    const float* __restrict__ slots, float* __restrict__ dwte,
                                                    int accumulate) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (v >= V) return;
  const int rs = seg_start[v], re = seg_end[v];
  float* dst = dwte + (long)v * C;
  if (rs < 0) {
    if (!accumulate)
      for (int col = lane * 8; col < C; col += 512) {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        Vec8<float>::store(dst + col, z);
      }
    return;
  }
  const int cs = rs / CHUNK, ce = (re - 1) / CHUNK;
  if (cs == ce) return;  // written by embed_chunk_k
  for (int col = lane * 8; col < C; col += 512) {
    float acc[8];
    Vec8<float>::load(slots + (long)(2 * cs + 1) * C + col, acc);
    for (int c = cs + 1; c <= ce; ++c) {
      float x[8];
      Vec8<float>::load(slots + (long)(2 * c) * C + col, x);
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
    if (accumulate) {
      float o[8];
      Vec8<float>::load(dst + col, o);
      for (int e = 0; e < 8; ++e) acc[e] += o[e];
    }
    Vec8<float>::store(dst + col, acc);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void embed_pos_k(int B, int TT, int C, int rows, const T* __restrict__ dx0,
                                                   float* __restrict__ dwpe, int accumulate) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)rows * C) return;
  const int t = (int)(idx / C), c = (int)(idx % C);
  float s = 0.0f;
  if (t < TT)
    for (int b = 0; b < B; ++b) s += to_f32(dx0[((long)b * TT + t) * C + c]);
  dwpe[idx] = accumulate ? dwpe[idx] + s : s;
}

struct EmbedWs {
  size_t sort, skeys, spos, seg_start, seg_end, slots, total;
  long P;  // keys sorted: N rounded up to a power of two
};

EmbedWs embed_ws_layout(int N, int V, int C) {
  EmbedWs w{};
  w.P = 2;
  while (w.P < N) w.P <<= 1;
  size_t o = 0;
  w.sort = o; o += align256((size_t)w.P * 8);
  w.skeys = o; o += align256((size_t)N * 4);
  w.spos = o; o += align256((size_t)N * 4);
  w.seg_start = o; o += align256((size_t)V * 4);
  w.seg_end = o; o += align256((size_t)V * 4);
  w.slots = o; o += align256((size_t)2 * cdiv(N, CHUNK) * C * 4);
  w.total = o;
  return w;
}

// Sorts the P keys at k ascending (the bitonic network above).
hipError_t bitonic_sort(uint64_t* k, long P, hipStream_t s) {
  const int n = (int)std::min<long>(P, SORT_TILE);
  const unsigned tiles = (unsigned)(P / n);
  hipLaunchKernelGGL(bitonic_tile_k, dim3(tiles), dim3(SORT_THREADS), 0, s, k, n, 2, n);
  for (long m = 2L * n; m <= P; m <<= 1) {
    for (long st = m >> 1; st >= n; st >>= 1)
      hipLaunchKernelGGL(bitonic_pass_k, dim3((unsigned)cdiv(P / 2, 256)), dim3(256), 0, s, k, P, m, st);
    hipLaunchKernelGGL(bitonic_tile_k, dim3(tiles), dim3(SORT_THREADS), 0, s, k, n, (int)m, (int)m);
  }
  return hipGetLastError();
}

}  // namespace

size_t embed_bwd_scratch_bytes(int N, int V) {
  // C-independent part plus slots sized for the widest supported row (2048)
  return embed_ws_layout(N, V, 2048).total;
}

hipError_t launch_embed_fwd(int dtype, int B, int T, int C, int V, const int32_t* ids, const void* wte,
                            const void* wpe, void* x0, hipStream_t s) {
  const int N = B * T;
  dim3 grid(cdiv(N, 4));
  if (dtype == 1)
    hipLaunchKernelGGL(embed_fwd_k<bf16>, grid, dim3(256), 0, s, N, T, C, V, ids, (const bf16*)wte, (const bf16*)wpe,
                       (bf16*)x0);
  else
    hipLaunchKernelGGL(embed_fwd_k<float>, grid, dim3(256), 0, s, N, T, C, V, ids, (const float*)wte,
                       (const float*)wpe, (float*)x0);
  return hipGetLastError();
}

hipError_t launch_embed_bwd(int dtype, int B, int T, int C, int V, int wpe_rows, const int32_t* ids,
                            const void* dx0, float* dwte, float* dwpe, int accumulate, void* scratch,
                            size_t scratch_bytes, hipStream_t s) {
  const int N = B * T;
  EmbedWs w = embed_ws_layout(N, V, C);
  if (scratch_bytes < w.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(scratch);
  uint64_t* sortk = reinterpret_cast<uint64_t*>(base + w.sort);
  int32_t* keys_out = reinterpret_cast<int32_t*>(base + w.skeys);
  int32_t* vals_out = reinterpret_cast<int32_t*>(base + w.spos);
  int32_t* seg_start = reinterpret_cast<int32_t*>(base + w.seg_start);
  int32_t* seg_end = reinterpret_cast<int32_t*>(base + w.seg_end);
  float* slots = reinterpret_cast<float*>(base + w.slots);
  hipLaunchKernelGGL(sort_keys_k, dim3((unsigned)cdiv(w.P, 256)), dim3(256), 0, s, N, (int)w.P, V, ids, sortk);
  hipLaunchKernelGGL(fill_i32_k, dim3(std::min(cdiv(V, 256), 1024)), dim3(256), 0, s, (long)V, seg_start, -1);
  hipLaunchKernelGGL(fill_i32_k, dim3(std::min(cdiv(V, 256), 1024)), dim3(256), 0, s, (long)V, seg_end, -1);
  hipError_t e = bitonic_sort(sortk, w.P, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_keys_k, dim3(cdiv(N, 256)), dim3(256), 0, s, N, sortk, keys_out, vals_out);
  hipLaunchKernelGGL(seg_bounds_k, dim3(cdiv(N, 256)), dim3(256), 0, s, N, V, keys_out, seg_start, seg_end);
  const int nchunk = cdiv(N, CHUNK);
  if (dtype == 1)
    hipLaunchKernelGGL(embed_chunk_k<bf16>, dim3(cdiv(nchunk, 4)), dim3(256), 0, s, N, C, V, keys_out, vals_out,
                       (const bf16*)dx0, seg_start, seg_end, dwte, slots, accumulate);
  else
    hipLaunchKernelGGL(embed_chunk_k<float>, dim3(cdiv(nchunk, 4)), dim3(256), 0, s, N, C, V, keys_out, vals_out,
                       (const float*)dx0, seg_start, seg_end, dwte, slots, accumulate);
  hipLaunchKernelGGL(embed_rows_k, dim3(cdiv(V, 4)), dim3(256), 0, s, V, C, seg_start, seg_end, slots, dwte,
                     accumulate);
  e = hipGetLastError();
  if (e != hipSuccess || !dwpe) return e;
  const long total = (long)wpe_rows * C;
  dim3 grid((unsigned)cdiv(total, 256));
  if (dtype == 1)
    hipLaunchKernelGGL(embed_pos_k<bf16>, grid, dim3(256), 0, s, B, T, C, wpe_rows, (const bf16*)dx0, dwpe,
                       accumulate);
  else
    hipLaunchKernelGGL(embed_pos_k<float>, grid, dim3(256), 0, s, B, T, C, wpe_rows, (const float*)dx0, dwpe,
                       accumulate);
  return hipGetLastError();
}
