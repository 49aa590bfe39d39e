// Row-block embedding kernel (bf16): for 64 token rows per work-group,
//   1. each row's sequence (binary search over the sequence offsets) and
//      position inside it;
//   2. x = LayerNorm_emb(E[id])            (token embedding, gain only)
//   3. qkv = x . W_qkv^T with RoPE on q and k, the first layer's attention
//      input (that layer has no attention pre-norm).
// The building blocks (row statistics, the QKV phase and its weight pipes)
// are those of jl_rowblock.h.
#include "jl_rowblock.h"

namespace jl {
namespace {
using namespace rowblock;

__global__ __launch_bounds__(512, 1) void embed_qkv_kernel(EmbedArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sA[RB * kWidth];  // 48 KB: x as bf16
  __shared__ __attribute__((aligned(16))) float sCos[RB * 32];   // 8 KB: RoPE rows of this block
  __shared__ __attribute__((aligned(16))) float sSin[RB * 32];   // 8 KB
  __shared__ float sRed[2][NW][RB];
  __shared__ int sPos[RB];
  __shared__ __attribute__((aligned(16))) bf16 sStage[NW * 4096];  // 64 KB: 8 KB per wave for the q/k/v stores
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = (a.rev ? gridDim.x - 1 - blockIdx.x : blockIdx.x) * RB;
  const int T = a.T;

  // 1. sequence and position of each row (rows past T repeat row T - 1)
  if (tid < RB) {
    const int row = min(row0 + tid, T - 1);
    int lo = 0, hi = a.n_seqs - 1;  // last b with seq_offsets[b] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.seq_offsets[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    const int p = row - a.seq_offsets[lo];
    sPos[tid] = p;
    if (row0 + tid < T) {
      a.pos[row] = p;
      a.tok_seq[row] = lo;
    }
  }

  // 2. embedding rows (wave w: columns 48 w .. 48 w + 47); an id outside the
  //    vocabulary reads row 0 and its output row is NaN
  f32x4 X[4][3];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = a.ids[min(row0 + 16 * i + r16, T - 1)];
    ok[i] = id >= 0 && id < kVocab;
    const float *e = a.emb + (size_t)(ok[i] ? id : 0) * kWidth + 48 * wave + 4 * g;
#pragma unroll
    for (int j = 0; j < 3; ++j) X[i][j] = *reinterpret_cast<const f32x4 *>(e + 16 * j);
  }
  __syncthreads();  // sPos
  stage_rope(sCos, sSin, a.rope_cos, a.rope_sin, tid, [&](int r) { return sPos[r]; });

  float mean[4], rstd[4];
  row_stats(X, sRed, lane, wave, mean, rstd);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * wave + 16 * j + 4 * g;
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(a.gain + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X[i][j][r] = ok[i] ? (X[i][j][r] - mean[i]) * rstd[i] * gm[r] : NAN;
      const int row = row0 + 16 * i + r16;
      if (row < T) *reinterpret_cast<f32x4 *>(a.x + (size_t)row * kWidth + col) = X[i][j];
      put4(sA, 16 * i + r16, col, KSD, X[i][j][0], X[i][j][1], X[i][j][2], X[i][j][3]);
    }
  }
  __syncthreads();

  // 3. the first layer's QKV with RoPE
  PipeO po;
  PipeI pi;
  Pipe2 p2;
  f32x4 H[4][4];
  qkv_phase<false>(a.Wqkv, nullptr, a.qkv_out, sCos, sSin, sA, po, pi, p2, H, X, lane, wave, row0, T,
                   sStage + wave * 4096);
}

}  // namespace

hipError_t launch_embed_qkv(const EmbedArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.n_seqs <= 0) return hipErrorInvalidValue;
  embed_qkv_kernel<<<(a.T + RB - 1) / RB, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace jl
