// Row-block layer kernel (bf16): everything of one encoder layer after its
// attention, plus the next layer's QKV, for 64 token rows per work-group.
//
// Per block, with its 64 rows resident in LDS and registers:
//   1. x += o . W_o^T                      (attention out-projection, residual)
//   2. u  = LayerNorm_mlp(x)               (row statistics across the 8 waves)
//   3. x += GEGLU(u . W_i^T) . W_out^T     (intermediate in chunks of 256
//                                           columns, never stored outside LDS)
//   4. either u' = LayerNorm_attn(next)(x); qkv = u' . W_qkv(next)^T with RoPE
//      on q and k (stored bf16 for the next attention),
//      or, after the last layer, h = LayerNorm_final(x) + type row (and, in
//      head mode, the first head layer's LayerNorm and biased in-projection).
//
// Waves 0-3 and 4-7 run the MLP and QKV phases in rotated orders, so that on
// each SIMD one wave's vector work (GEGLU, RoPE) overlaps its partner's
// matrix-core work.  Building blocks (weight pipes, fragment-order tiles, row
// statistics, the QKV phase) are in jl_rowblock.h.
#include "jl_rowblock.h"

namespace jl {
namespace {
using namespace rowblock;

// W_i chunk c (outputs 256 c .. 256 c + 64 NTI - 1, i.e. 128 NTI interleaved
// rows): wave w's (GELU group, gate group) pairs, groups 32 c + NTI w + j.
template <int NTI, int PD>
DI void start_wi(WPipe<NTI, PD> &w, const LayerArgs &a, int c, int lane, int wave) {
  int ng[NTI];
#pragma unroll
  for (int j = 0; j < NTI; ++j) ng[j] = 32 * c + NTI * wave + j;
  wp_start(w, a.Wi, KSD, ng, 0, lane);
}
// e4m3 W_i in units of 128 intermediate columns: unit u, wave w is the
// GELU/gate group pair 16 u + 2 w, + 1 (intermediate columns 128 u + 16 w ..
// + 15), so a unit's GEGLU output is 128 contiguous columns.
DI void start_wi8u(Pipe28 &w, const LayerArgs &a, int u, int lane, int wave) {
  const int ng[2] = {16 * u + 2 * wave, 16 * u + 2 * wave + 1};
  wp8_start(w, a.Wi8, ng, lane);
}
DI void scale_wi8u(f32x4 (&H)[4][4], const LayerArgs &a, int u, const float (&srow)[4], int lane, int wave) {
  const int ng[2] = {16 * u + 2 * wave, 16 * u + 2 * wave + 1};
  scale8<2>(H, ng, a.si, srow, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) H[i][1] *= 0.5f;  // the gate, halved as in the bf16 packing
}
// W_out k-steps of unit u (4 of them) for wave w's 48 output columns.
DI void start_wout_u(PipeO &w, const LayerArgs &a, int u, int lane, int wave) {
  const int ng[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
  wp_start(w, a.Wout, kGeglu / 32, ng, 4 * u, lane);
}
// W_out k-steps of chunk c for wave w's 48 output columns.
DI void start_wout(PipeO &w, const LayerArgs &a, int c, int lane, int wave) {
  const int ng[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
  wp_start(w, a.Wout, kGeglu / 32, ng, 8 * c, lane);
}
// gelu(z) * g for a gate value gh = g / 2 (the packed W_i carries the gate
// rows halved): gelu(z) = (z + |z| erf(|z| / sqrt 2)) / 2, erf from
// Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7), erf = 1 - t P(t) exp(-x^2),
// t = 1 / (1 + p x), x = |z| / sqrt 2, with 1 / sqrt 2 folded into p and the
// exponent.  12 vector operations and 2 transcendentals per value.
DI float geglu_half_gate(float z, float gh) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189450033013f, az, 1.0f));  // p / sqrt 2
  float q = fmaf(1.061405429f, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  q = q * t;
  const float e = __builtin_amdgcn_exp2f((z * z) * -0.72134752044448170f);  // exp(-z^2 / 2)
  const float u = fmaf(-az, q * e, az);                                     // |z| erf(|z| / sqrt 2)
  return (z + u) * gh;
}

// GEGLU of the pair (H[.][0], H[.][1]) into a unit buffer (fragment order,
// 64 x 128): wave w's columns 16 w .. 16 w + 15.
DI void geglu_unit(const f32x4 (&H)[4][4], bf16 *sHb, int lane, int wave) {
  const int r16 = lane & 15, g = lane >> 4;
  const int col = 16 * wave + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    put4(sHb, 16 * i + r16, col, 4, geglu_half_gate(H[i][0][0], H[i][1][0]), geglu_half_gate(H[i][0][1], H[i][1][1]),
         geglu_half_gate(H[i][0][2], H[i][1][2]), geglu_half_gate(H[i][0][3], H[i][1][3]));
}

// GEGLU of H[.][0, NTI) into the chunk buffer sHb (fragment order, 64 x 64 NTI).
template <int NTI>
DI void geglu(const f32x4 (&H)[4][4], bf16 *sHb, int lane, int wave) {
  constexpr int KS = 2 * NTI;  // k-steps of the chunk buffer
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int p = 0; p < NTI / 2; ++p) {
    const int col = 8 * NTI * wave + 16 * p + 4 * g;  // chunk-local output column
#pragma unroll
    for (int i = 0; i < 4; ++i)
      put4(sHb, 16 * i + r16, col, KS, geglu_half_gate(H[i][2 * p][0], H[i][2 * p + 1][0]),
           geglu_half_gate(H[i][2 * p][1], H[i][2 * p + 1][1]), geglu_half_gate(H[i][2 * p][2], H[i][2 * p + 1][2]),
           geglu_half_gate(H[i][2 * p][3], H[i][2 * p + 1][3]));
  }
}

// kHeadNext: after the last layer, continue into the first head layer's
// LayerNorm (with shift) and biased in-projection, without RoPE.
// kF8: W_i and the next encoder layer's QKV take e4m3 operands (their
// LayerNorm tiles coded per row into sA); the head's in-projection, the
// out-projection and W_out stay bf16.
template <bool kHeadNext, bool kF8>
__global__ __launch_bounds__(512, 1) void layer_kernel(LayerArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sA[RB * kWidth];  // 48 KB: o, then u, then u'
  __shared__ float sAmax[kF8 ? NW : 1][RB];                       // e4m3: partial row maxima
  uint8_t *sA8 = reinterpret_cast<uint8_t *>(sA);                 // e4m3: the coded u, then u'
  __shared__ __attribute__((aligned(16))) bf16 sH0[RB * 256];    // 32 KB: GEGLU chunk buffers,
  __shared__ __attribute__((aligned(16))) bf16 sH1[RB * 256];    // 32 KB: double-buffered
  __shared__ __attribute__((aligned(16))) float sCos[RB * 32];   // 8 KB: RoPE rows of this block
  __shared__ __attribute__((aligned(16))) float sSin[RB * 32];   // 8 KB
  __shared__ float sRed[2][NW][RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = (a.rev ? gridDim.x - 1 - blockIdx.x : blockIdx.x) * RB;
  const int T = a.T;
  const bool lead = wave < NW / 2;
  const bool next_layer = a.Wqkv_next != nullptr;

  // Every GEMM below runs on a weight pipe started during the previous GEMM's
  // last steps or before an epilogue, so none begins with an empty pipeline.
  // Waves take two pipe types in turn.
  PipeO po;
  PipeI pi;
  Pipe2 p2;
  Pipe28 pa8, pb8;  // e4m3 products (W_i units, QKV rotation halves)
  float srow[4];    // e4m3: scales of this lane's rows of the coded tile in sA8
  {
    const int ngo[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
    wp_start(po, a.Wo, KSD, ngo, 0, lane);  // needs nothing: first
  }

  // 1. attention output rows -> sA (fragment order), all 6 loads of a thread
  //    in flight before the first LDS store; the position of this thread's
  //    RoPE row, whose table rows are staged later, away from this phase
  constexpr int OL = RB * (kWidth / 8) / 512;  // 16-byte loads per thread
  static_assert(OL * 512 == RB * (kWidth / 8), "o staging");
  bf16x8 ov[OL];
#pragma unroll
  for (int q = 0; q < OL; ++q) {
    const int c = tid + 512 * q, r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    ov[q] = ldg8(a.o + (size_t)min(row0 + r, T - 1) * kWidth + k);
  }
  const bool rope_next = !kHeadNext && next_layer;
  const int rope_pos = rope_next ? a.pos[min(row0 + (tid >> 3), T - 1)] : 0;
#pragma unroll
  for (int q = 0; q < OL; ++q) {
    const int c = tid + 512 * q, r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    *reinterpret_cast<bf16x8 *>(&sA[afrag(r, k, KSD)]) = ov[q];
  }
  __syncthreads();

  // 2. X = x + o . W_o^T   (wave w: columns 48w .. 48w+47, 3 groups of 16)
  f32x4 X[4][3];
  zero(X);
  if constexpr (kF8) wp_run<KSD>(X, po, sA, lane, [&] { start_wi8u(pa8, a, 0, lane, wave); });
  else wp_run<KSD>(X, po, sA, lane, [&] { start_wi(pi, a, 0, lane, wave); });
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = min(row0 + 16 * i + r16, T - 1);
    const float *xr = a.x + (size_t)row * kWidth + 48 * wave + 4 * g;
#pragma unroll
    for (int j = 0; j < 3; ++j) X[i][j] += *reinterpret_cast<const f32x4 *>(xr + 16 * j);
  }

  // 3. u = LayerNorm_mlp(X) -> sA (the syncs in row_stats also retire every read of o)
  float mean[4], rstd[4];
  row_stats(X, sRed, lane, wave, mean, rstd);
  if constexpr (kF8) write_ln8<false>(X, a.mlp_norm, nullptr, mean, rstd, sAmax, sA8, srow, lane, wave);
  else write_ln<false>(X, a.mlp_norm, nullptr, mean, rstd, sA, lane, wave);
  __syncthreads();

  // 4. MLP: the 1,152 intermediate columns in 4 chunks of 256 and one of 128,
  //    chunk c's GEGLU output in buffer c % 2.  Step c (between barriers)
  //    completes chunk c's GEGLU and runs chunk c-1's W_out.  Waves 0-3 run
  //    [W_out(c-1), W_i(c), GEGLU(c)]; waves 4-7 run [GEGLU(c), W_out(c-1),
  //    W_i(c+1)], keeping the W_i accumulators across the barrier.  On every
  //    SIMD one wave's GEGLU arithmetic then overlaps its partner's
  //    matrix-core work.  X receives the chunks in order.
  f32x4 H[4][4];
  if constexpr (kF8) {
    // e4m3: the 1,152 intermediate columns in 9 units of 128, unit u's GEGLU
    // output in buffer u % 2 (fragment order, 4 k-steps).  Waves 0-3 run
    // step u as [W_out(u-1), W_i(u), GEGLU(u)], waves 4-7 as [GEGLU(u),
    // W_out(u-1), W_i(u+1)], keeping the W_i accumulators across the
    // barrier, so that on every SIMD one wave's GEGLU overlaps its partner's
    // products; a unit's product keeps 32 accumulators live.
    constexpr int NU = kGeglu / 128;
    auto run_in = [&](int u) {
      zero_cols<2>(H);
      wp8_run(H, pa8, sA8, lane, NoNext());
      scale_wi8u(H, a, u, srow, lane, wave);
      pin_acc<2>(H);  // the products complete here, not sunk past the barrier into the GEGLU
    };
    if (lead) {
      run_in(0);  // its pipe started during the out-projection
      start_wout_u(po, a, 0, lane, wave);
      geglu_unit(H, sH0, lane, wave);
      __syncthreads();
#pragma unroll 1
      for (int u = 1; u < NU; ++u) {
        bf16 *prev = (u & 1) ? sH0 : sH1, *cur = (u & 1) ? sH1 : sH0;
        wp_run<4>(X, po, prev, lane, [&] { start_wi8u(pa8, a, u, lane, wave); });
        run_in(u);
        start_wout_u(po, a, u, lane, wave);
        geglu_unit(H, cur, lane, wave);
        __syncthreads();
      }
    } else {
      run_in(0);
      start_wi8u(pa8, a, 1, lane, wave);
      geglu_unit(H, sH0, lane, wave);
      run_in(1);
      start_wout_u(po, a, 0, lane, wave);
      __syncthreads();
#pragma unroll 1
      for (int u = 1; u < NU - 1; ++u) {
        bf16 *prev = (u & 1) ? sH0 : sH1, *cur = (u & 1) ? sH1 : sH0;
        geglu_unit(H, cur, lane, wave);
        wp_run<4>(X, po, prev, lane, [&] { start_wi8u(pa8, a, u + 1, lane, wave); });
        run_in(u + 1);
        start_wout_u(po, a, u, lane, wave);
        __syncthreads();
      }
      geglu_unit(H, sH0, lane, wave);  // unit 8 into buffer 0, W_out(7) from buffer 1
      wp_run<4>(X, po, sH1, lane, NoNext());
      start_wout_u(po, a, NU - 1, lane, wave);
      __syncthreads();
    }
  } else if (lead) {
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, NoNext());
    start_wout(po, a, 0, lane, wave);
    geglu<4>(H, sH0, lane, wave);
    __syncthreads();
#pragma unroll 1
    for (int c = 1; c < 4; ++c) {
      bf16 *prev = (c & 1) ? sH0 : sH1, *cur = (c & 1) ? sH1 : sH0;
      wp_run<8>(X, po, prev, lane, [&] { start_wi(pi, a, c, lane, wave); });
      zero_cols<4>(H);
      wp_run<KSD>(H, pi, sA, lane, NoNext());
      start_wout(po, a, c, lane, wave);
      geglu<4>(H, cur, lane, wave);
      __syncthreads();
    }
    wp_run<8>(X, po, sH1, lane, [&] { start_wi(p2, a, 4, lane, wave); });
    zero_cols<2>(H);
    wp_run<KSD>(H, p2, sA, lane, NoNext());
    start_wout(po, a, 4, lane, wave);
    geglu<2>(H, sH0, lane, wave);
    __syncthreads();
  } else {
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, NoNext());
    start_wi(pi, a, 1, lane, wave);
    geglu<4>(H, sH0, lane, wave);
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, NoNext());
    start_wout(po, a, 0, lane, wave);
    __syncthreads();
#pragma unroll 1
    for (int c = 1; c < 3; ++c) {
      bf16 *prev = (c & 1) ? sH0 : sH1, *cur = (c & 1) ? sH1 : sH0;
      geglu<4>(H, cur, lane, wave);
      wp_run<8>(X, po, prev, lane, [&] { start_wi(pi, a, c + 1, lane, wave); });
      zero_cols<4>(H);
      wp_run<KSD>(H, pi, sA, lane, NoNext());
      start_wout(po, a, c, lane, wave);
      __syncthreads();
    }
    geglu<4>(H, sH1, lane, wave);
    wp_run<8>(X, po, sH0, lane, [&] { start_wi(p2, a, 4, lane, wave); });
    zero_cols<2>(H);
    wp_run<KSD>(H, p2, sA, lane, NoNext());
    start_wout(po, a, 3, lane, wave);
    __syncthreads();
    geglu<2>(H, sH0, lane, wave);
    wp_run<8>(X, po, sH1, lane, NoNext());
    start_wout(po, a, 4, lane, wave);
    __syncthreads();
  }
  // last W_out, with the RoPE table rows of this block's positions (the next
  // layer's q and k) in flight; they reach LDS after it, and the barriers of
  // the row statistics below publish them
  f32x4 rc, rs;
  if (rope_next) {
    const int q = (tid & 7) * 4;
    rc = *reinterpret_cast<const f32x4 *>(a.rope_cos_next + rope_pos * 32 + q);
    rs = *reinterpret_cast<const f32x4 *>(a.rope_sin_next + rope_pos * 32 + q);
  }
  wp_run<4>(X, po, sH0, lane, NoNext());
  if (rope_next) {
    const int r = tid >> 3, q = (tid & 7) * 4;
    *reinterpret_cast<f32x4 *>(&sCos[r * 32 + q]) = rc;
    *reinterpret_cast<f32x4 *>(&sSin[r * 32 + q]) = rs;
  }

  // 5. after the last layer: h = LayerNorm_final(X) + type row, into x (in
  //    head mode also kept in X for the head's first layer); otherwise the
  //    residual stream
  if constexpr (kHeadNext) {
    row_stats(X, sRed, lane, wave, mean, rstd);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 16 * i + r16;
      const float *tr = a.type_rows + (size_t)a.qtype[a.tok_seq[min(row, T - 1)]] * kWidth;
      float *xr = a.x + (size_t)row * kWidth;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int col = 48 * wave + 16 * j + 4 * g;
        const f32x4 gm = *reinterpret_cast<const f32x4 *>(a.final_norm + col);
        const f32x4 ty = *reinterpret_cast<const f32x4 *>(tr + col);
#pragma unroll
        for (int r = 0; r < 4; ++r) X[i][j][r] = (X[i][j][r] - mean[i]) * rstd[i] * gm[r] + ty[r];
        if (row < T) *reinterpret_cast<f32x4 *>(xr + col) = X[i][j];
      }
    }
  } else {
    if (!next_layer && a.final_norm != nullptr) {
      row_stats(X, sRed, lane, wave, mean, rstd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 16 * i + r16;
        if (row >= T) continue;
        const float *tr = a.type_rows + (size_t)a.qtype[a.tok_seq[row]] * kWidth;
        float *xr = a.x + (size_t)row * kWidth;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int col = 48 * wave + 16 * j + 4 * g;
          const f32x4 gm = *reinterpret_cast<const f32x4 *>(a.final_norm + col);
          const f32x4 ty = *reinterpret_cast<const f32x4 *>(tr + col);
          f32x4 h;
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = (X[i][j][r] - mean[i]) * rstd[i] * gm[r] + ty[r];
          *reinterpret_cast<f32x4 *>(xr + col) = h;
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 16 * i + r16;
      if (row >= T) continue;
      float *xr = a.x + (size_t)row * kWidth + 48 * wave + 4 * g;
#pragma unroll
      for (int j = 0; j < 3; ++j) *reinterpret_cast<f32x4 *>(xr + 16 * j) = X[i][j];
    }
    if (!next_layer) return;  // residual only (hidden-state diagnostics)
  }

  // 6. next layer: u' = LayerNorm_attn(next)(X) -> sA; its QKV (encoder
  //    layers rotate q and k; the head's first layer adds the bias).  The
  //    GEGLU buffers are free now: each wave stages its q/k/v stores through
  //    8 KB of them.
  row_stats(X, sRed, lane, wave, mean, rstd);
  if constexpr (kF8 && !kHeadNext) {
    PipeO8 po8;
    write_ln8<false>(X, a.attn_norm_next, nullptr, mean, rstd, sAmax, sA8, srow, lane, wave);
    __syncthreads();
    qkv_phase8(a.Wqkv8_next, a.sqkv_next, a.qkv_out, sCos, sSin, sA8, srow, po8, pa8, pb8, H, X, lane, wave, row0,
               T, (wave < NW / 2 ? sH0 : sH1) + (wave & 3) * 4096);
  } else {
    write_ln<kHeadNext>(X, a.attn_norm_next, a.attn_shift_next, mean, rstd, sA, lane, wave);
    __syncthreads();
    qkv_phase<kHeadNext>(a.Wqkv_next, a.qkv_bias_next, a.qkv_out, sCos, sSin, sA, po, pi, p2, H, X, lane, wave,
                         row0, T, (wave < NW / 2 ? sH0 : sH1) + (wave & 3) * 4096);
  }
}

}  // namespace

hipError_t launch_layer(const LayerArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const dim3 grid((a.T + RB - 1) / RB);
  const bool f8 = a.Wi8 != nullptr;
  if (f8 && (a.si == nullptr || (a.Wqkv_next != nullptr && a.qkv_bias_next == nullptr &&
                                 (a.Wqkv8_next == nullptr || a.sqkv_next == nullptr))))
    return hipErrorInvalidValue;  // e4m3 codes without their scales, or a next layer without codes
  if (a.qkv_bias_next != nullptr) {
    if (f8) layer_kernel<true, true><<<grid, 512, 0, s>>>(a);
    else layer_kernel<true, false><<<grid, 512, 0, s>>>(a);
  } else {
    if (f8) layer_kernel<false, true><<<grid, 512, 0, s>>>(a);
    else layer_kernel<false, false><<<grid, 512, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace jl
