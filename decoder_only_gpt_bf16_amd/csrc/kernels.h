// Internal launch interface between the C-ABI host code and the kernels.
#pragma once
#include "common.h"

// ---------------------------------------------------------------------------
// GEMM: C(m, n) = sum_k A(m, k) * B(n, k), fp32 accumulation.
//   A row-major [M, lda] with k contiguous        (a_kmaj = false), or
//             [K, lda] with m contiguous          (a_kmaj = true);
//   B row-major [N, ldb] with k contiguous        (b_kmaj = false), or
//             [K, ldb] with n contiguous          (b_kmaj = true).
// Forward Linear: A = activations, B = weight [out, in] (both k-contiguous).
// Input gradient dX = dY W: B = W given as [K = out, N = in] (b_kmaj).
// Weight gradient dW = dY^T X: A = dY as [K = tokens, M = out] (a_kmaj),
//   B = X as [K = tokens, N = in] (b_kmaj).
// ---------------------------------------------------------------------------
enum EpiKind {
  EPI_STORE = 0,      // out(T) = acc (+ bias[n]) (+ resid[m, n])
  EPI_GELU = 1,       // u = acc + bias[n]; out(T) = gelu'(u) (skipped when out is NULL); out2(T) = gelu(u)
  EPI_GELU_BWD = 2,   // out(T) = acc * aux[m, n] (aux = the stored gelu'(u))
  EPI_F32 = 3,        // out(f32) = acc (+ out if accumulate)
  EPI_XENT_STATS = 4, // per (row, 128-col block): max and sum exp; target logit
  EPI_XENT_GRAD = 5,  // out(T) = (exp(acc - lse[m]) - [n + col_offset == tgt[m]]) * scale (* roww[m])
  EPI_QKNORM = 6,     // fused QKV (N = 3C, head_dim 128): out(T) = acc (+ bias), then RoPE and
                      // QK-norm on the q and k heads; 1 / rms of each into qk_rstd [2][M][H]
};

struct GemmParams {
  const void* A;
  const void* B;
  long lda, ldb;
  int M, N, K;
  int k_split;            // K elements handled per blockIdx.z
  int tiles_m, tiles_n;
  uint32_t a_bytes, b_bytes;  // bytes of A and B covered by their buffer loads
  // epilogue
  void* out;
  long ldc;
  long split_stride;      // elements between per-split partial outputs
  const void* bias;
  const void* resid;
  long ldr;
  void* out2;
  const void* aux;
  long ldaux;
  int accumulate;
  // cross-entropy epilogues
  const int32_t* tgt;
  int col_offset;
  float2* part;           // [M, part_ld] (max, sum exp) partials
  int part_ld;
  int part_off;
  float* ztgt;            // [M] target logits
  const float* lse;       // [M]
  float scale;
  const float* roww;      // [M] per-row weight of EPI_XENT_GRAD, or nullptr
  // fused RoPE / QK-norm epilogue
  const float2* qk_cs;    // [T][64] (cos, sin)
  float* qk_rstd;
  int qk_T, qk_rope, qk_norm;
  float qk_eps;
  // FP8 operands: quantizer scale arrays of A and B (element 2 = 1 / scale)
  const float* f8_sa;
  const float* f8_sb;
};

struct GemmDesc {
  const void* A; long lda; bool a_kmaj;
  const void* B; long ldb; bool b_kmaj;
  int M, N, K;
  int epi;
  void* out; long ldc;
  const void* bias;
  const void* resid; long ldr;
  void* out2;
  const void* aux; long ldaux;
  int accumulate;
  const int32_t* tgt; int col_offset; float2* part; int part_ld; int part_off;
  float* ztgt; const float* lse; float scale; const float* roww;
  const float2* qk_cs; float* qk_rstd; int qk_T, qk_rope, qk_norm; float qk_eps;
  const float* f8_sa; const float* f8_sb;  // launch_gemm_fp8: operands' scale arrays
};

// Bytes of split-K scratch launch_gemm may use for this problem (0 if none).
size_t gemm_split_scratch_bytes(const GemmDesc& d, int dtype);
// Columns per cross-entropy partial of the bf16 MFMA path.
int xent_part_cols();
// Launch; `ws` provides split-K scratch of gemm_split_scratch_bytes().
hipError_t launch_gemm(const GemmDesc& d, int dtype, void* ws, hipStream_t s);
// The same GEMM with FP8 operands (byte codes, k contiguous on both sides,
// K, lda and ldb multiples of 16), dequantized by f8_sa[2] * f8_sb[2] before
// the epilogue.  mode 1: A and B E4M3; mode 2: A E5M2, B E4M3.
hipError_t launch_gemm_fp8(const GemmDesc& d, int mode, void* ws, hipStream_t s);
size_t gemm_fp8_split_scratch_bytes(const GemmDesc& d);
// Up to GEMM_GROUP_MAX independent fp32-output (EPI_F32) problems with both
// operands k-major and one K (the weight gradients of a block) as one
// stream-K launch plus a fixed-order fixup of the tiles split between
// blocks; falls back to one launch_gemm each.  `ws` must hold
// gemm_group_scratch_bytes() bytes.
constexpr int GEMM_GROUP_MAX = 4;
size_t gemm_group_scratch_bytes(const GemmDesc* d, int n, int dtype);
// The same grouping for FP8 weight gradients: A = dY codes in E5M2, B = X
// codes in E4M3, both k contiguous (launch_gemm_fp8's operand rules, mode 2);
// falls back to one launch_gemm_fp8 each.  `ws` must hold
// gemm_group_fp8_scratch_bytes() bytes.
size_t gemm_group_fp8_scratch_bytes(const GemmDesc* d, int n);
// bf16 transposes dst[c][r] = src[r][c] ([rows][cols] row-major in, [cols][rows]
// out), up to TRANSPOSE_MAX in one launch; rows and cols multiples of 8
constexpr int TRANSPOSE_MAX = 4;
struct TransposeDesc {
  const void* src;
  void* dst;
  int rows, cols;
};
hipError_t launch_transpose(const TransposeDesc* d, int n, hipStream_t s);

// The same jobs as a kernel argument: blocks [start[j], start[j + 1]) of a
// launch cover matrix j in 64-row x 256-column tiles.  A thread moves one
// 8 x 8 block: 8 row vectors of 16 bytes in, transposed in registers (halves
// of 32-bit words regrouped), 8 row vectors of the transpose out.  A wave
// covers 64 x 64 elements as 8 x 8 such blocks, so that both its loads and
// its stores are whole 128-byte rows of 8 lanes.  256 threads per block.
struct TransposeJobs {
  const bf16* src[TRANSPOSE_MAX];
  bf16* dst[TRANSPOSE_MAX];
  int rows[TRANSPOSE_MAX], cols[TRANSPOSE_MAX], tiles_c[TRANSPOSE_MAX];
  int start[TRANSPOSE_MAX + 1];
  int n;
};
// fills J from d[0 .. n); returns the number of blocks the jobs need
inline int make_transpose_jobs(const TransposeDesc* d, int n, TransposeJobs& J) {
  J.n = n;
  J.start[0] = 0;
  for (int i = 0; i < n; ++i) {
    J.src[i] = static_cast<const bf16*>(d[i].src);
    J.dst[i] = static_cast<bf16*>(d[i].dst);
    J.rows[i] = d[i].rows;
    J.cols[i] = d[i].cols;
    J.tiles_c[i] = (d[i].cols + 255) / 256;
    J.start[i + 1] = J.start[i] + (d[i].rows + 63) / 64 * J.tiles_c[i];
  }
  return J.start[n];
}
// block `bid` (< the count above) of the jobs
__device__ __forceinline__ void transpose_block(const TransposeJobs& J, int bid) {
  int j = 0;
  while (j + 1 < J.n && bid >= J.start[j + 1]) ++j;
  const int tid = bid - J.start[j];
  const int R = J.rows[j], Cc = J.cols[j];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = (tid / J.tiles_c[j]) * 64 + 8 * (lane >> 3);
  const int c = (tid % J.tiles_c[j]) * 256 + 64 * wave + 8 * (lane & 7);
  if (r >= R || c >= Cc) return;
  const bf16* src = J.src[j] + (long)r * Cc + c;
  uint4 in[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) in[i] = *reinterpret_cast<const uint4*>(src + (long)i * Cc);
  bf16* dst = J.dst[j] + (long)c * R + r;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    // output row q (source column q): word k pairs source rows 2k and 2k + 1
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = reinterpret_cast<const uint32_t*>(&in[2 * k])[q >> 1];
      const uint32_t b = reinterpret_cast<const uint32_t*>(&in[2 * k + 1])[q >> 1];
      w[k] = (q & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<uint4*>(dst + (long)q * R) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}
hipError_t launch_gemm_group(const GemmDesc* d, int n, int dtype, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_gemm_group_fp8(const GemmDesc* d, int n, void* ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------------------
// Norms, embeddings, attention, cross-entropy, reductions.
// ---------------------------------------------------------------------------
// rope (optional): the same launch also writes that RoPE table.
hipError_t launch_norm_fwd(int dtype, int kind, int N, int C, const void* x, const void* w,
                           const void* b, float eps, void* y, float* stats, hipStream_t s,
                           const RopeJob* rope = nullptr);
// dx = norm_bwd(dy) (+ resid); column partial sums of dy*xhat and dy into
// colpart [2][nblk][C] (when want_cols), reduced by launch_colsum_finish.
hipError_t launch_norm_bwd(int dtype, int kind, int N, int C, const void* x, const void* w,
                           const void* dy, const void* resid, float eps, void* dx,
                           float* colpart, int want_cols, hipStream_t s);
int norm_bwd_blocks(int N);
hipError_t launch_colsum_finish(int C, int nblk, const float* part, float* out, int accumulate,
                                hipStream_t s);
// Several such reductions in one launch: out_j[c] (+)= sum over b < nblk_j of
// part_j[b][c], each in the same fixed order as launch_colsum_finish.
constexpr int COLSUM_JOBS_MAX = 8;
struct ColsumJob {
  const float* part;
  int nblk, C;
  float* out;
};
hipError_t launch_colsum_finish_jobs(const ColsumJob* jobs, int n, int accumulate, hipStream_t s);
// Per-block column partials of a [N, C] matrix (storage dtype, leading
// dimension ld) for the finish above (bias gradients): part
// [colsum_part_blocks(N)][C] fp32.
int colsum_part_blocks(int N);
size_t colsum_scratch_bytes(int N, int C);
hipError_t launch_colsum_part(int dtype, int N, int C, long ld, const void* x, float* part, hipStream_t s);

// ids outside [0, V) give a zero token embedding (no out-of-range read).
hipError_t launch_embed_fwd(int dtype, int B, int T, int C, int V, const int32_t* ids, const void* wte,
                            const void* wpe, void* x0, hipStream_t s);
size_t embed_bwd_scratch_bytes(int N, int V);
// dwpe [wpe_rows, C] (rows >= T receive 0) or NULL.  ids outside [0, V)
// contribute nothing.
hipError_t launch_embed_bwd(int dtype, int B, int T, int C, int V, int wpe_rows, const int32_t* ids,
                            const void* dx0, float* dwte, float* dwpe, int accumulate, void* scratch,
                            size_t scratch_bytes, hipStream_t s);

// RoPE angle table: cs[t * (D/2) + i] = (cos, sin)(t * base^(-2i/D)).
// In place on the q and k thirds of qkv [N, 3C]: RoPE then QK-norm; saves
// 1/rms of q and k per (row, head) into rstd [2][N][H] when qk_norm.
hipError_t launch_qk_fwd(int dtype, int B, int T, int H, int D, int rope, int qk_norm, float eps,
                         const float2* cs, void* qkv, float* rstd, hipStream_t s);
// In place on dq, dk thirds of dqkv: QK-norm backward (needs the normalised
// q, k from qkv and rstd), then the inverse rotation.
hipError_t launch_qk_bwd(int dtype, int B, int T, int H, int D, int rope, int qk_norm,
                         const float2* cs, const void* qkv, const float* rstd, void* dqkv,
                         hipStream_t s);
// Causal attention forward: q, k, v inside qkv [N, 3C]; o [N, C]; lse fp32 [B, H, T].
// qk_norm != 0 promises RMS-normalised q and k (|q|, |k| <= sqrt(D)), which
// lets the softmax use a fixed shift instead of a running maximum.
// window > 0: query i attends to keys i - window + 1 .. i only (0: full causal).
// side[0 .. nside): bf16 transposes that ride in the same launch (MFMA path:
// extra blocks after the attention's; other paths: a launch of their own
// after it), nside <= TRANSPOSE_MAX.
hipError_t launch_attn_fwd(int dtype, int B, int T, int H, int D, int qk_norm, int window, const void* qkv, void* o,
                           float* lse, const TransposeDesc* side, int nside, hipStream_t s);
// delta[b, h, t] = sum_d dO * O (fp32 [B, H, T]).
hipError_t launch_attn_delta(int dtype, int B, int T, int H, int D, const void* o, const void* dO,
                             float* delta, hipStream_t s);
// Attention backward into the dk | dv thirds and the dq third of dqkv [N, 3C].
// QK-norm / RoPE backward folded into the stores of dQ and dK (MFMA path).
struct QkBwd {
  int rope, qk_norm;
  int N;                // B * T
  const float2* cs;     // RoPE table [T][D / 2] of (cos, sin)
  const float* rstd;    // saved 1 / rms of q then k, [2][N][H]
};
// MFMA path (attn_mfma_supported): run dQ first; it also writes delta for
// the dK/dV pass, and both apply the QK-norm / RoPE backward of qk.  Other
// paths: delta comes from launch_attn_delta, qk is ignored and
// launch_qk_bwd follows.
hipError_t launch_attn_bwd_dkdv(int dtype, int B, int T, int H, int D, int window, const void* qkv, const void* dO,
                                const float* lse, const float* delta, void* dqkv, const QkBwd& qk, hipStream_t s);
hipError_t launch_attn_bwd_dq(int dtype, int B, int T, int H, int D, int window, const void* qkv, const void* o,
                              const void* dO,
                              const float* lse, float* delta, void* dqkv, const QkBwd& qk, hipStream_t s);
bool attn_mfma_supported(int dtype, int D);

// Cross-entropy reductions.
// Combine per-row partials into lse, nats = lse - ztgt (NaN for a target
// outside [0, V), whose ztgt no chunk wrote), block loss partials.
// w (optional): per-token weights of the loss sum; a token of weight 0
// contributes nothing (also when its target is out of range).
hipError_t launch_xent_finish(int N, int P, int V, const float2* part, const int32_t* tgt, const float* ztgt,
                              const float* w, float* lse, float* nats, float* loss_part, hipStream_t s);
hipError_t launch_loss_sum(int nblk, const float* loss_part, float scale, float* loss,
                           hipStream_t s);
int xent_finish_blocks(int N);
// Generic path: running row statistics over a materialised fp32 logit chunk.
hipError_t launch_xent_rows_stats(int N, int Vc, int v0, const float* z, long ldz,
                                  const int32_t* tgt, float2* run, float* ztgt, int first,
                                  hipStream_t s);
hipError_t launch_xent_rows_grad(int dtype, int N, int Vc, int v0, const float* z, long ldz,
                                 const int32_t* tgt, const float* lse, float scale, const float* w, void* dz,
                                 long lddz, hipStream_t s);
hipError_t launch_f32_to(int dtype, long n, const float* src, void* dst, hipStream_t s);

// targets outside [0, V) count as zero-byte tokens.
hipError_t launch_bpb(int N, int V, const float* nats, const int32_t* targets, const int32_t* token_bytes,
                      double* sum_nats, int64_t* sum_bytes, hipStream_t s);

// AdamW with global-norm clipping over a set of fp32 tensors (optim.hip).
constexpr int OPT_TABLE = 32;  // tensors per launch
struct OptTensor {
  float* p;
  const float* g;
  float* m;
  float* v;
  void* p16;  // bf16 copy of the updated parameter, or nullptr
  long n;
  int decay;
};
long adamw_chunks(const OptTensor* t, int count);
size_t adamw_ws_bytes(const OptTensor* t, int count);
// max_norm <= 0: no clipping.  norm_out (device, optional) receives the global
// gradient norm before clipping.  ws: adamw_ws_bytes bytes.
hipError_t launch_adamw(const OptTensor* t, int count, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int step, float max_norm, float* norm_out, void* ws,
                        hipStream_t s);
// The allocation-free variant's scratch: a device array of this many chunk
// partials (plus 256 bytes) per GPU; adamw_noalloc_scratch gives its address
// on the current device.
constexpr long ADAMW_NOALLOC_MAX_CHUNKS = 131072;
hipError_t adamw_noalloc_scratch(void** ptr);

// FP8 (fp8.hip).  Formats: OCP E4M3 and E5M2.
constexpr int FP8_E4M3 = 0, FP8_E5M2 = 1;
long fp8_amax_parts(long n);
// scal (device float[3]) <- scale, amax, 1 / scale; q <- codes; part: fp8_amax_parts(n) floats
hipError_t launch_fp8_quantize(long n, const void* x, int fmt, void* q, float* scal, float* part, hipStream_t s);
// Up to Q2D_MAX bf16 matrices x [R][Cc] (Cc a multiple of 16) quantized to
// one format, each with its own scale: scal as above; q [R][Cc] codes (or
// NULL) and qT [Cc][ldT] transposed codes (or NULL; ldT >= R a multiple of
// 64, columns R .. ldT - 1 zero).  part: fp8_q2d_parts(n) floats.
constexpr int Q2D_MAX = 4;
struct Fp8Q2d {
  const void* x;
  void* q;
  void* qT;
  long ldT;
  int R, Cc;
  float* scal;
};
constexpr long fp8_q2d_parts(int n) { return 1024L * n; }
hipError_t launch_fp8_quantize_2d(const Fp8Q2d* d, int n, int fmt, float* part, hipStream_t s);
// out (bf16, ldc) = A B^T * scal_a[2] * scal_b[2]; A [M][lda], B [N][ldb] codes, k contiguous
hipError_t launch_fp8_gemm(int M, int N, int K, const void* A, long lda, int fa, const float* scal_a, const void* B,
                           long ldb, int fb, const float* scal_b, void* out, long ldc, hipStream_t s);
