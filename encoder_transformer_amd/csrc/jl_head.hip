// Row-block head-layer kernel (bf16): one head layer (torch pre-norm encoder
// layer, biases everywhere) after its attention, for 64 token rows per
// work-group, with the weight pipes and fragment-order LDS tiles of
// jl_rowblock.h:
//   1. x += o . W_o^T + b_o
//   2. u  = LayerNorm_2(x)                          (gain and shift)
//   3. x += relu(u . W_1^T + b_1) . W_2^T + b_2     (1,536 hidden columns in 6
//                                                    chunks of 256, LDS only)
//   4. store x; then the next head layer's u' = LayerNorm_1(next)(x) and its
//      keys and values u' . W_kv^T + b_kv (bf16, [T, 768]).
// The ReLU epilogue is a few operations per value, so all 8 waves run the
// same order: W_1 chunk, epilogue, barrier, W_2 chunk.
#include "jl_rowblock.h"

namespace jl {
namespace {
using namespace rowblock;

constexpr int KSF = kHeadFfn / 32;  // 48 k-steps over the head's hidden width
constexpr int kHeadChunks = kHeadFfn / 256;

// W_1 chunk c (hidden columns 256 c .. 256 c + 255): wave w's groups 16 c + 2 w + j.
DI void start_w1(Pipe2 &w, const HeadArgs &a, int c, int lane, int wave) {
  const int ng[2] = {16 * c + 2 * wave, 16 * c + 2 * wave + 1};
  wp_start(w, a.W1, KSD, ng, 0, lane);
}
// W_2 k-steps of chunk c for wave w's 48 output columns.
DI void start_w2(PipeO &w, const HeadArgs &a, int c, int lane, int wave) {
  const int ng[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
  wp_start(w, a.W2, KSF, ng, 8 * c, lane);
}

// relu(H + b_1) of chunk c into the chunk buffer sHb (fragment order, 64 x 256):
// wave w holds chunk-local columns 32 w .. 32 w + 31.
DI void relu_store(const f32x4 (&H)[4][2], const float *b1, int c, bf16 *sHb, int lane, int wave) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = 32 * wave + 16 * j + 4 * g;
    const f32x4 b = *reinterpret_cast<const f32x4 *>(b1 + 256 * c + col);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      put4(sHb, 16 * i + r16, col, 8, fmaxf(H[i][j][0] + b[0], 0.f), fmaxf(H[i][j][1] + b[1], 0.f),
           fmaxf(H[i][j][2] + b[2], 0.f), fmaxf(H[i][j][3] + b[3], 0.f));
  }
}

__global__ __launch_bounds__(512, 1) void head_kernel(HeadArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sA[RB * kWidth];  // 48 KB: o, then u, then u'
  __shared__ __attribute__((aligned(16))) bf16 sH0[RB * 256];    // 32 KB: ReLU chunk buffers,
  __shared__ __attribute__((aligned(16))) bf16 sH1[RB * 256];    // 32 KB: double-buffered
  __shared__ float sRed[2][NW][RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = (a.rev ? gridDim.x - 1 - blockIdx.x : blockIdx.x) * RB;
  const int T = a.T;

  PipeO po;
  PipeI pi;
  Pipe2 p2;
  {
    const int ngo[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
    wp_start(po, a.Wo, KSD, ngo, 0, lane);
  }
  // attention output rows -> sA (fragment order), all loads of a thread in
  // flight before its first LDS store
  constexpr int OL = RB * (kWidth / 8) / 512;
  bf16x8 ov[OL];
#pragma unroll
  for (int q = 0; q < OL; ++q) {
    const int c = tid + 512 * q, r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    ov[q] = ldg8(a.o + (size_t)min(row0 + r, T - 1) * kWidth + k);
  }
#pragma unroll
  for (int q = 0; q < OL; ++q) {
    const int c = tid + 512 * q, r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    *reinterpret_cast<bf16x8 *>(&sA[afrag(r, k, KSD)]) = ov[q];
  }
  __syncthreads();

  // 1. X = x + o . W_o^T + b_o   (wave w: columns 48w .. 48w+47)
  f32x4 X[4][3];
  zero(X);
  wp_run<KSD>(X, po, sA, lane, [&] { start_w1(p2, a, 0, lane, wave); });
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * wave + 16 * j + 4 * g;
    const f32x4 b = *reinterpret_cast<const f32x4 *>(a.bo + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(row0 + 16 * i + r16, T - 1);
      X[i][j] = *reinterpret_cast<const f32x4 *>(a.x + (size_t)row * kWidth + col) + (X[i][j] + b);
    }
  }

  // 2. u = LayerNorm_2(X) -> sA (the syncs in row_stats retire every read of o)
  float mean[4], rstd[4];
  row_stats(X, sRed, lane, wave, mean, rstd);
  write_ln<true>(X, a.n2_w, a.n2_b, mean, rstd, sA, lane, wave);
  __syncthreads();

  // 3. feed-forward: chunk c's ReLU output in buffer c % 2; W_2(c) runs after
  //    the barrier that publishes it, while the next chunk's W_1 fragments
  //    are already in flight
  f32x4 H[4][2];
#pragma unroll 1
  for (int c = 0; c < kHeadChunks; ++c) {
    bf16 *buf = (c & 1) ? sH1 : sH0;
    zero(H);
    wp_run<KSD>(H, p2, sA, lane, NoNext());
    start_w2(po, a, c, lane, wave);
    relu_store(H, a.b1, c, buf, lane, wave);
    __syncthreads();
    wp_run<8>(X, po, buf, lane, [&] {
      if (c + 1 < kHeadChunks) start_w1(p2, a, c + 1, lane, wave);
    });
  }

  // 4. X += b_2 -> x; the next layer's keys and values
  const bool kv = a.Wkv != nullptr;
  if (kv) {
    const int ng[4] = {4 * wave, 4 * wave + 1, 4 * wave + 2, 4 * wave + 3};
    wp_start(pi, a.Wkv, KSD, ng, 0, lane);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * wave + 16 * j + 4 * g;
    const f32x4 b = *reinterpret_cast<const f32x4 *>(a.b2 + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      X[i][j] += b;
      const int row = row0 + 16 * i + r16;
      if (row < T) *reinterpret_cast<f32x4 *>(a.x + (size_t)row * kWidth + col) = X[i][j];
    }
  }
  if (!kv) return;
  row_stats(X, sRed, lane, wave, mean, rstd);
  write_ln<true>(X, a.nk_w, a.nk_b, mean, rstd, sA, lane, wave);
  __syncthreads();
  // 768 columns = 48 groups, 6 per wave: first wave w's 4 groups 4w ..
  // (columns 64 w .., one 128-byte line of each row), then 2 groups of the
  // last 256 columns (waves 2v and 2v + 1 share a line).  Each line of kv is
  // then written whole within one pass, not in pieces far apart in time.
  const int ng4[4] = {4 * wave, 4 * wave + 1, 4 * wave + 2, 4 * wave + 3};
  const int ng2[2] = {32 + 2 * wave, 32 + 2 * wave + 1};
  f32x4 K4[4][4];
  zero(K4);
  wp_run<KSD>(K4, pi, sA, lane, [&] { wp_start(p2, a.Wkv, KSD, ng2, 0, lane); });
  bias_store<4>(K4, ng4, a.bkv, a.kv_out, 2 * kWidth, lane, row0, T);
  zero(H);
  wp_run<KSD>(H, p2, sA, lane, NoNext());
  bias_store<2>(H, ng2, a.bkv, a.kv_out, 2 * kWidth, lane, row0, T);
}

}  // namespace

hipError_t launch_head_layer(const HeadArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  head_kernel<<<(a.T + RB - 1) / RB, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace jl
