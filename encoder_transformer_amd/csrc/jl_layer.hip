// Row-block layer kernel (bf16): everything of one encoder layer after its
// attention, plus the next layer's QKV, for 64 token rows per work-group.
//
// Per block, with its 64 rows resident in LDS and registers:
//   1. x += o . W_o^T                      (attention out-projection, residual)
//   2. u  = LayerNorm_mlp(x)               (row statistics across the 8 waves)
//   3. x += GEGLU(u . W_i^T) . W_out^T     (intermediate in chunks of 128 columns,
//                                           never stored outside LDS)
//   4. either u' = LayerNorm_attn(next)(x); qkv = u' . W_qkv(next)^T with RoPE
//      on q and k (stored bf16 for the next attention),
//      or, after the last layer, h = LayerNorm_final(x) + type row.
//
// 512 threads = 8 waves, two per SIMD, so one wave's vector work (LayerNorm,
// GEGLU, RoPE) overlaps the other's matrix-core work.  The weights stream
// from L2 straight into matrix-core fragments: at load they are pre-packed so
// that each (16 output columns x 32 k) block is the 1 KB a wave consumes, one
// coalesced load, issued 4 k-steps ahead.  The activations (LayerNorm output,
// GEGLU chunk) sit in LDS in fragment order.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16 with the weight fragment as the A
// operand and the activation fragment as B, so the accumulator is C^T: lane
// (r16 + 16 g) holds row r16 of the 16-row sub-tile and the 4 consecutive
// columns 4g .. 4g+3 of the 16-column sub-tile.  Row statistics then reduce
// over 4 lanes, and every epilogue access is a 16-byte (FP32) or 8-byte (bf16)
// vector.
#include "jl_device.h"

// No FMA contraction: unrolled code handles each row of a tile in its own
// instruction sequence, and a contraction the compiler applies to some of
// those sequences and not to others would make a row's rounding depend on
// its place in the tile, and so on how the batch was packed.
#pragma clang fp contract(off)

namespace jl {
namespace {
using namespace dev;

constexpr int RB = kLayerRows;    // 64 rows per work-group
constexpr int NW = 8;             // waves per work-group
constexpr int KSD = kWidth / 32;  // 12 k-steps over the model width

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 ldg8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x8 lds8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Element offset of (row, k) in a fragment-ordered [64 x (32 * ksteps)] tile:
// block (row / 16, k / 32) of 64 lanes x 8 elements, lane (row % 16) + 16 * ((k % 32) / 8).
__device__ inline int afrag(int row, int k, int ksteps) {
  return ((row >> 4) * ksteps + (k >> 5)) * 512 + ((row & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// 4 consecutive columns (k .. k+3, k % 4 == 0) of one row as bf16 into a fragment tile.
__device__ inline void put4(bf16 *tile, int row, int k, int ksteps, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4 *>(tile + afrag(row, k, ksteps)) = v;
}

// acc[i][j] += (A_tile(LDS, 64 x 32*KSTEPS) . Wp^T)^T sub-tiles for this wave's
// NT groups of 16 output columns (group ng[j]), k-steps ks0 .. ks0+KSTEPS-1 of
// Wp.  B fragments for steps s .. s+PD-1 are in flight; each register is
// consumed in place and reloaded right after, so nothing forces an early wait.
template <int NT, int KSTEPS, int PD>
__device__ inline void gemm_rows(f32x4 (&acc)[4][NT], const bf16 *sAt, const bf16 *__restrict__ Wp,
                                 int w_ksteps, const int (&ng)[NT], int ks0, int lane) {
  static_assert(KSTEPS % PD == 0 && PD % 2 == 0, "k-steps: a multiple of an even prefetch depth");
  const bf16 *wp[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wp[j] = Wp + ((size_t)ng[j] * w_ksteps + ks0) * 512 + lane * 8;
  const bf16 *ap = sAt + lane * 8;
  bf16x8 fb[PD][NT], fa[2][4];
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int j = 0; j < NT; ++j) fb[p][j] = ldg8(wp[j] + p * 512);
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = lds8(ap + (i * KSTEPS) * 512);
#pragma unroll 1
  for (int s0 = 0; s0 < KSTEPS; s0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int s = s0 + p;
      if (s + 1 < KSTEPS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[(p + 1) & 1][i] = lds8(ap + (i * KSTEPS + s + 1) * 512);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[p][j], fa[p & 1][i], acc[i][j], 0, 0, 0);
      if (s + PD < KSTEPS) {
#pragma unroll
        for (int j = 0; j < NT; ++j) fb[p][j] = ldg8(wp[j] + (s + PD) * 512);
      }
    }
  }
}

template <int NT>
__device__ inline void zero(f32x4 (&acc)[4][NT]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Row statistics of the 64 x 384 tile X: wave w holds columns 48w .. 48w+47 as
// 3 sub-tiles; lane (r16 + 16 g) holds row 16 i + r16, columns 16 j + 4 g + r.
// Two passes (mean, then the mean of squared deviations), reduced over the 4
// lane groups and then over the 8 waves through LDS.
__device__ inline void row_stats(const f32x4 (&X)[4][3], float (*sRed)[RB], int lane, int wave,
                                 float (&mean)[4], float (&rstd)[4]) {
  const int r16 = lane & 15, g = lane >> 4;
  float part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j) s += (X[i][j][0] + X[i][j][1]) + (X[i][j][2] + X[i][j][3]);
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    part[i] = s;
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sRed[wave][16 * i + r16] = part[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * i + r16;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += sRed[w][row];
    mean[i] = t * (1.0f / kWidth);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = X[i][j][r] - mean[i];
        s += d * d;
      }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    part[i] = s;
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sRed[wave][16 * i + r16] = part[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * i + r16;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += sRed[w][row];
    rstd[i] = rsqrtf(t * (1.0f / kWidth) + kLnEps);
  }
  __syncthreads();
}

// sA = bf16(gain * (X - mean) * rstd), fragment order over the full width.
__device__ inline void write_ln(const f32x4 (&X)[4][3], const float *__restrict__ gain, const float (&mean)[4],
                                const float (&rstd)[4], bf16 *sA, int lane, int wave) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * wave + 16 * j + 4 * g;
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(gain + col);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      put4(sA, 16 * i + r16, col, KSD, (X[i][j][0] - mean[i]) * rstd[i] * gm[0],
           (X[i][j][1] - mean[i]) * rstd[i] * gm[1], (X[i][j][2] - mean[i]) * rstd[i] * gm[2],
           (X[i][j][3] - mean[i]) * rstd[i] * gm[3]);
  }
}

// q/k columns head_col .. head_col+63 of one head for this block's rows, RoPE
// applied: NT = 4 covers the whole head, NT = 2 the half `half` (d in
// 16 half .. 16 half + 15 and its partners d + 32).
template <int NT>
__device__ inline void rope_heads(const bf16 *sA, const float *sCos, const float *sSin, const LayerArgs &a,
                                  int head_col, int half, int lane, int row0, int T) {
  const int r16 = lane & 15, g = lane >> 4;
  f32x4 H[4][NT];
  zero(H);
  int ng[NT];
  if (NT == 4) {
#pragma unroll
    for (int j = 0; j < NT; ++j) ng[j] = head_col / 16 + j;
  } else {
    ng[0] = head_col / 16 + half;
    ng[1] = head_col / 16 + half + 2;
  }
  gemm_rows<NT, KSD, (NT == 4 ? 2 : 4)>(H, sA, a.Wqkv_next, KSD, ng, 0, lane);
#pragma unroll
  for (int jp = 0; jp < NT / 2; ++jp) {
    const int d0 = 16 * (NT == 4 ? jp : half) + 4 * g;  // this lane's rotation indices d0 .. d0+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 16 * i + r16, row = row0 + rl;
      if (row >= T) continue;
      const f32x4 cs = *reinterpret_cast<const f32x4 *>(sCos + rl * 32 + d0);
      const f32x4 sn = *reinterpret_cast<const f32x4 *>(sSin + rl * 32 + d0);
      bf16x4 lo, hi;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = H[i][jp][r], x1 = H[i][jp + NT / 2][r];  // partner d + 32
        lo[r] = (bf16)(x0 * cs[r] - x1 * sn[r]);
        hi[r] = (bf16)(x1 * cs[r] + x0 * sn[r]);
      }
      bf16 *q = a.qkv_out + (size_t)row * (3 * kWidth) + head_col + d0;
      *reinterpret_cast<bf16x4 *>(q) = lo;
      *reinterpret_cast<bf16x4 *>(q + 32) = hi;
    }
  }
}

// One MLP chunk: outputs 256 c .. 256 c + 64 PAIRS (PAIRS = 4: 256 outputs,
// PAIRS = 2: the last 128).  Wave w computes outputs 256 c + 16 PAIRS/2 ... as
// PAIRS/2 (GELU, gate) group pairs, writes GEGLU into sH, then every wave adds
// sH . W_out^T over the chunk's k-range into its 48 columns of X.
template <int NTI>
__device__ inline void mlp_chunk(f32x4 (&X)[4][3], const bf16 *sA, bf16 *sH, const LayerArgs &a, int c, int lane,
                                 int wave) {
  constexpr int OUT = 8 * 8 * NTI;  // outputs in this chunk: 256 (NTI 4) or 128 (NTI 2)
  constexpr int KS = OUT / 32;      // W_out k-steps of the chunk
  const int r16 = lane & 15, g = lane >> 4;
  f32x4 H[4][NTI];
  zero(H);
  int ng[NTI];
#pragma unroll
  for (int j = 0; j < NTI; ++j) ng[j] = 32 * c + NTI * wave + j;  // 512 W_i rows = 32 groups per full chunk
  gemm_rows<NTI, KSD, (NTI == 4 ? 2 : 4)>(H, sA, a.Wi, KSD, ng, 0, lane);
#pragma unroll
  for (int p = 0; p < NTI / 2; ++p) {
    const int col = 8 * NTI * wave + 16 * p + 4 * g;  // chunk-local output column
#pragma unroll
    for (int i = 0; i < 4; ++i)
      put4(sH, 16 * i + r16, col, KS, gelu_erf(H[i][2 * p][0]) * H[i][2 * p + 1][0],
           gelu_erf(H[i][2 * p][1]) * H[i][2 * p + 1][1], gelu_erf(H[i][2 * p][2]) * H[i][2 * p + 1][2],
           gelu_erf(H[i][2 * p][3]) * H[i][2 * p + 1][3]);
  }
  __syncthreads();
  {
    const int ngo[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
    gemm_rows<3, KS, 4>(X, sH, a.Wout, kGeglu / 32, ngo, 8 * c, lane);
  }
  __syncthreads();  // sH is rewritten by the next chunk
}

__global__ __launch_bounds__(512, 1) void layer_kernel(LayerArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sA[RB * kWidth];  // 48 KB: o, then u, then u'
  __shared__ __attribute__((aligned(16))) bf16 sH[RB * 256];     // 32 KB: one GEGLU chunk
  __shared__ __attribute__((aligned(16))) float sCos[RB * 32];   // 8 KB: RoPE rows of this block
  __shared__ __attribute__((aligned(16))) float sSin[RB * 32];   // 8 KB
  __shared__ float sRed[NW][RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * RB;
  const int T = a.T;

  // 1. attention output rows -> sA (fragment order); the RoPE table rows of
  //    this block's positions -> LDS, for the next layer's q and k
  for (int c = tid; c < RB * (kWidth / 8); c += 512) {
    const int r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    const int src = min(row0 + r, T - 1);
    *reinterpret_cast<bf16x8 *>(&sA[afrag(r, k, KSD)]) = ldg8(a.o + (size_t)src * kWidth + k);
  }
  if (a.Wqkv_next != nullptr) {
    for (int c = tid; c < RB * 8; c += 512) {  // 64 rows x 8 float4 of each table
      const int r = c >> 3, q = (c & 7) * 4;
      const int p = a.pos[min(row0 + r, T - 1)];
      *reinterpret_cast<f32x4 *>(&sCos[r * 32 + q]) = *reinterpret_cast<const f32x4 *>(a.rope_cos_next + p * 32 + q);
      *reinterpret_cast<f32x4 *>(&sSin[r * 32 + q]) = *reinterpret_cast<const f32x4 *>(a.rope_sin_next + p * 32 + q);
    }
  }
  __syncthreads();

  // 2. X = x + o . W_o^T   (wave w: columns 48w .. 48w+47, 3 groups of 16)
  f32x4 X[4][3];
  zero(X);
  {
    const int ng[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
    gemm_rows<3, KSD, 4>(X, sA, a.Wo, KSD, ng, 0, lane);
  }
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
  write_ln(X, a.mlp_norm, mean, rstd, sA, lane, wave);
  __syncthreads();

  // 4. MLP: the 1,152 intermediate columns in 4 chunks of 256 and one of 128.
  //    A chunk of n outputs is 2n interleaved W_i rows; wave w takes its
  //    share as (GELU group, gate group) pairs of the same 16 outputs.
  mlp_chunk<4>(X, sA, sH, a, 0, lane, wave);
  mlp_chunk<4>(X, sA, sH, a, 1, lane, wave);
  mlp_chunk<4>(X, sA, sH, a, 2, lane, wave);
  mlp_chunk<4>(X, sA, sH, a, 3, lane, wave);
  mlp_chunk<2>(X, sA, sH, a, 4, lane, wave);

  // 5. after the last layer: h = LayerNorm_final(X) + type row, into x
  if (a.Wqkv_next == nullptr && a.final_norm != nullptr) {
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
  // otherwise store the residual stream
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 16 * i + r16;
    if (row >= T) continue;
    float *xr = a.x + (size_t)row * kWidth + 48 * wave + 4 * g;
#pragma unroll
    for (int j = 0; j < 3; ++j) *reinterpret_cast<f32x4 *>(xr + 16 * j) = X[i][j];
  }
  if (a.Wqkv_next == nullptr) return;  // residual only (hidden-state diagnostics)

  // 6. next layer: u' = LayerNorm_attn(X) -> sA; qkv = u' . W_qkv^T
  row_stats(X, sRed, lane, wave, mean, rstd);
  write_ln(X, a.attn_norm_next, mean, rstd, sA, lane, wave);
  __syncthreads();
  // q and k (12 heads): heads 0-7 one per wave (4 groups: d 0-15, 16-31 and
  // their RoPE partners 32-47, 48-63), then heads 8-11 two waves each (the
  // wave's half h: groups h and h + 2).
  rope_heads<4>(sA, sCos, sSin, a, 64 * wave, 0, lane, row0, T);
  rope_heads<2>(sA, sCos, sSin, a, 512 + 64 * (wave >> 1), wave & 1, lane, row0, T);
  // v: 384 columns, wave w columns 48w .. 48w+47 (X's registers are free again)
  zero(X);
  {
    const int ng[3] = {48 + 3 * wave, 48 + 3 * wave + 1, 48 + 3 * wave + 2};
    gemm_rows<3, KSD, 4>(X, sA, a.Wqkv_next, KSD, ng, 0, lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 16 * i + r16;
    if (row >= T) continue;
    bf16 *v = a.qkv_out + (size_t)row * (3 * kWidth) + 2 * kWidth + 48 * wave + 4 * g;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      bf16x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (bf16)X[i][j][r];
      *reinterpret_cast<bf16x4 *>(v + 16 * j) = t;
    }
  }
}

}  // namespace

hipError_t launch_layer(const LayerArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  layer_kernel<<<(a.T + RB - 1) / RB, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace jl
