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
//      or, after the last layer, h = LayerNorm_final(x) + type row.
//
// 512 threads = 8 waves, two per SIMD.  Waves 0-3 and 4-7 run the MLP and
// QKV phases in rotated orders, so that on each SIMD one wave's vector work
// (GEGLU, RoPE) overlaps its partner's matrix-core work.  The weights stream
// from L2 straight into matrix-core fragments: at load they are pre-packed so
// that each (16 output columns x 32 k) block is the 1 KB a wave consumes, one
// coalesced buffer load; every GEMM runs on a "weight pipe" whose first
// k-steps were issued during the previous GEMM or before an epilogue.  The
// activations (LayerNorm output, GEGLU chunk) sit in LDS in fragment order.
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

#define DI __device__ __attribute__((always_inline)) inline

constexpr int RB = kLayerRows;    // 64 rows per work-group
constexpr int NW = 8;             // waves per work-group
constexpr int KSD = kWidth / 32;  // 12 k-steps over the model width

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

DI bf16x8 ldg8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
DI bf16x8 lds8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Element offset of (row, k) in a fragment-ordered [64 x (32 * ksteps)] tile:
// block (row / 16, k / 32) of 64 lanes x 8 elements, lane (row % 16) + 16 * ((k % 32) / 8).
DI int afrag(int row, int k, int ksteps) {
  return ((row >> 4) * ksteps + (k >> 5)) * 512 + ((row & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// 4 consecutive columns (k .. k+3, k % 4 == 0) of one row as bf16 into a fragment tile.
DI void put4(bf16 *tile, int row, int k, int ksteps, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4 *>(tile + afrag(row, k, ksteps)) = v;
}

// Raw buffer resource over packed weights: loads take a per-lane byte offset
// in a VGPR and the k-step offset as a scalar or immediate, so streaming them
// costs no vector address arithmetic.
DI __amdgpu_buffer_rsrc_t weight_rsrc(const bf16 *W) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16 *>(W), (short)0, 0x7fffffff, 0x00020000);
}
DI bf16x8 ldw(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// A weight pipe: PD k-steps of a wave's NT fragment columns in flight.
template <int NT, int PD>
struct WPipe {
  const bf16 *W;
  int vo[NT];
  bf16x8 fb[PD][NT];
};

// Issue the first PD k-steps of the fragments of groups ng[j] (k-steps ks0 ..)
// of a packed weight with w_ksteps k-steps per group.
template <int NT, int PD>
DI void wp_start(WPipe<NT, PD> &w, const bf16 *Wp, int w_ksteps, const int (&ng)[NT], int ks0, int lane) {
  w.W = Wp;
  const __amdgpu_buffer_rsrc_t rw = weight_rsrc(Wp);
#pragma unroll
  for (int j = 0; j < NT; ++j) w.vo[j] = ((ng[j] * w_ksteps + ks0) * 64 + lane) * 16;
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int j = 0; j < NT; ++j) w.fb[p][j] = ldw(rw, w.vo[j], p * 1024);
}

struct NoNext {
  DI void operator()() const {}
};

// acc[i][j] += (A_tile(LDS, 64 x 32*KSTEPS) . W^T)^T for a started pipe: each
// fragment register is reloaded right after the MFMAs that read it;
// activation fragments are double-buffered one step ahead.  `next()` runs at
// the start of the last PD steps, once every load of this GEMM is issued: it
// starts the wave's next pipe, so that GEMM begins with its fragments in
// flight.  Fully unrolled.
template <int KSTEPS, int NT, int PD, int NTA, class Next>
DI void wp_run(f32x4 (&acc)[4][NTA], WPipe<NT, PD> &w, const bf16 *sAt, int lane, Next next) {
  static_assert(NT <= NTA, "accumulator columns");
  static_assert(PD <= KSTEPS, "prefetch depth");
  const __amdgpu_buffer_rsrc_t rw = weight_rsrc(w.W);
  const bf16 *ap = sAt + lane * 8;
  bf16x8 fa[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = lds8(ap + (i * KSTEPS) * 512);
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int p = s % PD;
    if (s == KSTEPS - PD) next();
    if (s + 1 < KSTEPS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[(s + 1) & 1][i] = lds8(ap + (i * KSTEPS + s + 1) * 512);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.fb[p][j], fa[s & 1][i], acc[i][j], 0, 0, 0);
    if (s + PD < KSTEPS) {
#pragma unroll
      for (int j = 0; j < NT; ++j) w.fb[p][j] = ldw(rw, w.vo[j], (s + PD) * 1024);
    }
    // keep each reload right behind the MFMAs that free its registers: the
    // scheduler would otherwise sink the reloads towards the next wait
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NT>
DI void zero(f32x4 (&acc)[4][NT]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Row statistics of the 64 x 384 tile X: wave w holds columns 48w .. 48w+47 as
// 3 sub-tiles; lane (r16 + 16 g) holds row 16 i + r16, columns 16 j + 4 g + r.
// Two passes (mean, then the mean of squared deviations), reduced over the 4
// lane groups and then over the 8 waves through LDS.
DI void row_stats(const f32x4 (&X)[4][3], float (*sRed)[RB], int lane, int wave,
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

// sA = bf16(gain * (X - mean) * rstd [+ shift]), fragment order over the full width.
template <bool kShift>
DI void write_ln(const f32x4 (&X)[4][3], const float *__restrict__ gain, const float *__restrict__ shift,
                 const float (&mean)[4], const float (&rstd)[4], bf16 *sA, int lane, int wave) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * wave + 16 * j + 4 * g;
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(gain + col);
    f32x4 sh = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kShift) sh = *reinterpret_cast<const f32x4 *>(shift + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = (X[i][j][r] - mean[i]) * rstd[i] * gm[r];
        if constexpr (kShift) v[r] = v[r] + sh[r];
      }
      put4(sA, 16 * i + r16, col, KSD, v[0], v[1], v[2], v[3]);
    }
  }
}

// Pipe types: out-projection, W_out and v (3 groups); W_i chunks of 256 and
// the whole-head q/k (4 groups); the last W_i chunk and the half-head q/k (2).
constexpr int PDO = 3, PDI = 2, PD2 = 4;
using PipeO = WPipe<3, PDO>;
using PipeI = WPipe<4, PDI>;
using Pipe2 = WPipe<2, PD2>;

// W_i chunk c (outputs 256 c .. 256 c + 64 NTI - 1, i.e. 128 NTI interleaved
// rows): wave w's (GELU group, gate group) pairs, groups 32 c + NTI w + j.
template <int NTI, int PD>
DI void start_wi(WPipe<NTI, PD> &w, const LayerArgs &a, int c, int lane, int wave) {
  int ng[NTI];
#pragma unroll
  for (int j = 0; j < NTI; ++j) ng[j] = 32 * c + NTI * wave + j;
  wp_start(w, a.Wi, KSD, ng, 0, lane);
}
// W_out k-steps of chunk c for wave w's 48 output columns.
DI void start_wout(PipeO &w, const LayerArgs &a, int c, int lane, int wave) {
  const int ng[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
  wp_start(w, a.Wout, kGeglu / 32, ng, 8 * c, lane);
}
// Next layer's q/k of one whole head (wave w: head w) or of half a head
// (heads 8-11, two waves each: groups half and half + 2), and v (wave w:
// columns 48 w .. 48 w + 47).
DI void ng_qk_whole(int (&ng)[4], int wave) {
#pragma unroll
  for (int j = 0; j < 4; ++j) ng[j] = 4 * wave + j;
}
DI void ng_qk_half(int (&ng)[2], int wave) {
  const int base = 32 + 4 * (wave >> 1), half = wave & 1;
  ng[0] = base + half;
  ng[1] = base + half + 2;
}
DI void ng_v(int (&ng)[3], int wave) {
#pragma unroll
  for (int j = 0; j < 3; ++j) ng[j] = 48 + 3 * wave + j;
}
DI void start_qk_whole(PipeI &w, const LayerArgs &a, int lane, int wave) {
  int ng[4];
  ng_qk_whole(ng, wave);
  wp_start(w, a.Wqkv_next, KSD, ng, 0, lane);
}
DI void start_qk_half(Pipe2 &w, const LayerArgs &a, int lane, int wave) {
  int ng[2];
  ng_qk_half(ng, wave);
  wp_start(w, a.Wqkv_next, KSD, ng, 0, lane);
}
DI void start_v(PipeO &w, const LayerArgs &a, int lane, int wave) {
  int ng[3];
  ng_v(ng, wave);
  wp_start(w, a.Wqkv_next, KSD, ng, 0, lane);
}

template <int NTA>
DI void zero_cols(f32x4 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NTA; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// RoPE on q/k accumulators and store: NT = 4 holds a whole head (columns
// head_col .. head_col + 63, groups d 0-15, 16-31, 32-47, 48-63), NT = 2 the
// half `half` (groups d 16 half .. and d 32 + 16 half ..).  Rotation pairs
// are (d, d + 32).
template <int NT>
DI void rope_store(const f32x4 (&H)[4][4], const float *sCos, const float *sSin, const LayerArgs &a,
                   int head_col, int half, int lane, int row0, int T) {
  const int r16 = lane & 15, g = lane >> 4;
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

// v accumulators (wave w: columns 48 w .. 48 w + 47) to bf16.
DI void v_store(const f32x4 (&V)[4][3], const LayerArgs &a, int lane, int wave, int row0, int T) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 16 * i + r16;
    if (row >= T) continue;
    bf16 *v = a.qkv_out + (size_t)row * (3 * kWidth) + 2 * kWidth + 48 * wave + 4 * g;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      bf16x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (bf16)V[i][j][r];
      *reinterpret_cast<bf16x4 *>(v + 16 * j) = t;
    }
  }
}

// Biased projection columns to bf16 rows of `out` (row stride `stride`):
// accumulator column j holds output columns 16 ng[j] .. 16 ng[j] + 15.
template <int NT, int NTA>
DI void bias_store(const f32x4 (&H)[4][NTA], const int (&ng)[NT], const float *bias, bf16 *out, int stride,
                   int lane, int row0, int T) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int col = 16 * ng[j] + 4 * g;
    const f32x4 b = *reinterpret_cast<const f32x4 *>(bias + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 16 * i + r16;
      if (row >= T) continue;
      bf16x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (bf16)(H[i][j][r] + b[r]);
      *reinterpret_cast<bf16x4 *>(out + (size_t)row * stride + col) = t;
    }
  }
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
template <bool kHeadNext>
__global__ __launch_bounds__(512, 1) void layer_kernel(LayerArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sA[RB * kWidth];  // 48 KB: o, then u, then u'
  __shared__ __attribute__((aligned(16))) bf16 sH0[RB * 256];    // 32 KB: GEGLU chunk buffers,
  __shared__ __attribute__((aligned(16))) bf16 sH1[RB * 256];    // 32 KB: double-buffered
  __shared__ __attribute__((aligned(16))) float sCos[RB * 32];   // 8 KB: RoPE rows of this block
  __shared__ __attribute__((aligned(16))) float sSin[RB * 32];   // 8 KB
  __shared__ float sRed[NW][RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * RB;
  const int T = a.T;
  const bool lead = wave < NW / 2;
  const bool next_layer = a.Wqkv_next != nullptr;

  // Every GEMM below runs on a weight pipe started during the previous GEMM's
  // last steps or before an epilogue, so none begins with an empty pipeline.
  // Waves take two pipe types in turn.
  PipeO po;
  PipeI pi;
  Pipe2 p2;
  {
    const int ngo[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
    wp_start(po, a.Wo, KSD, ngo, 0, lane);  // needs nothing: first
  }

  // 1. attention output rows -> sA (fragment order); the RoPE table rows of
  //    this block's positions -> LDS, for the next layer's q and k
  for (int c = tid; c < RB * (kWidth / 8); c += 512) {
    const int r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    const int src = min(row0 + r, T - 1);
    *reinterpret_cast<bf16x8 *>(&sA[afrag(r, k, KSD)]) = ldg8(a.o + (size_t)src * kWidth + k);
  }
  if (!kHeadNext && next_layer) {
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
  wp_run<KSD>(X, po, sA, lane, [&] { start_wi(pi, a, 0, lane, wave); });
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
  write_ln<false>(X, a.mlp_norm, nullptr, mean, rstd, sA, lane, wave);
  __syncthreads();

  // 4. MLP: the 1,152 intermediate columns in 4 chunks of 256 and one of 128,
  //    chunk c's GEGLU output in buffer c % 2.  Step c (between barriers)
  //    completes chunk c's GEGLU and runs chunk c-1's W_out.  Waves 0-3 run
  //    [W_out(c-1), W_i(c), GEGLU(c)]; waves 4-7 run [GEGLU(c), W_out(c-1),
  //    W_i(c+1)], keeping the W_i accumulators across the barrier.  On every
  //    SIMD one wave's GEGLU arithmetic then overlaps its partner's
  //    matrix-core work.  X receives the chunks in order.
  f32x4 H[4][4];
  if (lead) {
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
  // last W_out
  wp_run<4>(X, po, sH0, lane, NoNext());

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

  // 6. next layer: u' = LayerNorm_attn(next)(X) -> sA; qkv = u' . W_qkv^T.
  //    q and k (12 heads): heads 0-7 one per wave, heads 8-11 two waves each;
  //    v: 48 columns per wave.  Waves 0-3 take [whole head, half head, v],
  //    waves 4-7 [half head, v, whole head], so epilogues overlap
  //    matrix-core work.  Encoder layers rotate q and k; the head's first
  //    layer adds the in-projection bias instead.
  row_stats(X, sRed, lane, wave, mean, rstd);
  write_ln<kHeadNext>(X, a.attn_norm_next, a.attn_shift_next, mean, rstd, sA, lane, wave);
  __syncthreads();
  const int half_col = 512 + 64 * (wave >> 1), half = wave & 1;
  int ngw[4], ngh[2], ngv[3];
  ng_qk_whole(ngw, wave);
  ng_qk_half(ngh, wave);
  ng_v(ngv, wave);
  constexpr int QS = 3 * kWidth;
  if (lead) {
    start_qk_whole(pi, a, lane, wave);
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, [&] { start_qk_half(p2, a, lane, wave); });
    if constexpr (kHeadNext) bias_store<4>(H, ngw, a.qkv_bias_next, a.qkv_out, QS, lane, row0, T);
    else rope_store<4>(H, sCos, sSin, a, 64 * wave, 0, lane, row0, T);
    zero_cols<2>(H);
    wp_run<KSD>(H, p2, sA, lane, [&] { start_v(po, a, lane, wave); });
    if constexpr (kHeadNext) bias_store<2>(H, ngh, a.qkv_bias_next, a.qkv_out, QS, lane, row0, T);
    else rope_store<2>(H, sCos, sSin, a, half_col, half, lane, row0, T);
    zero(X);
    wp_run<KSD>(X, po, sA, lane, NoNext());
    if constexpr (kHeadNext) bias_store<3>(X, ngv, a.qkv_bias_next, a.qkv_out, QS, lane, row0, T);
    else v_store(X, a, lane, wave, row0, T);
  } else {
    start_qk_half(p2, a, lane, wave);
    zero_cols<2>(H);
    wp_run<KSD>(H, p2, sA, lane, [&] { start_v(po, a, lane, wave); });
    if constexpr (kHeadNext) bias_store<2>(H, ngh, a.qkv_bias_next, a.qkv_out, QS, lane, row0, T);
    else rope_store<2>(H, sCos, sSin, a, half_col, half, lane, row0, T);
    zero(X);
    wp_run<KSD>(X, po, sA, lane, [&] { start_qk_whole(pi, a, lane, wave); });
    if constexpr (kHeadNext) bias_store<3>(X, ngv, a.qkv_bias_next, a.qkv_out, QS, lane, row0, T);
    else v_store(X, a, lane, wave, row0, T);
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, NoNext());
    if constexpr (kHeadNext) bias_store<4>(H, ngw, a.qkv_bias_next, a.qkv_out, QS, lane, row0, T);
    else rope_store<4>(H, sCos, sSin, a, 64 * wave, 0, lane, row0, T);
  }
}

// ---------------------------------------------------------------------------
// Head layer (torch pre-norm encoder layer, biases everywhere) after its
// attention, for 64 token rows per work-group, with the same weight pipes and
// fragment-order LDS tiles as the encoder layer:
//   1. x += o . W_o^T + b_o
//   2. u  = LayerNorm_2(x)                          (gain and shift)
//   3. x += relu(u . W_1^T + b_1) . W_2^T + b_2     (1,536 hidden columns in 6
//                                                    chunks of 256, LDS only)
//   4. store x; then the next head layer's u' = LayerNorm_1(next)(x) and its
//      keys and values u' . W_kv^T + b_kv (bf16, [T, 768]).
// The ReLU epilogue is a few operations per value, so all 8 waves run the
// same order: W_1 chunk, epilogue, barrier, W_2 chunk.

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
  __shared__ float sRed[NW][RB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * RB;
  const int T = a.T;

  PipeO po;
  PipeI pi;
  Pipe2 p2;
  {
    const int ngo[3] = {3 * wave, 3 * wave + 1, 3 * wave + 2};
    wp_start(po, a.Wo, KSD, ngo, 0, lane);
  }
  for (int c = tid; c < RB * (kWidth / 8); c += 512) {
    const int r = c / (kWidth / 8), k = (c % (kWidth / 8)) * 8;
    const int src = min(row0 + r, T - 1);
    *reinterpret_cast<bf16x8 *>(&sA[afrag(r, k, KSD)]) = ldg8(a.o + (size_t)src * kWidth + k);
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
    const int ng[4] = {6 * wave, 6 * wave + 1, 6 * wave + 2, 6 * wave + 3};
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
  // 768 columns = 48 groups, 6 per wave: 4 on one pipe, 2 on the other
  const int ng4[4] = {6 * wave, 6 * wave + 1, 6 * wave + 2, 6 * wave + 3};
  const int ng2[2] = {6 * wave + 4, 6 * wave + 5};
  f32x4 K4[4][4];
  zero(K4);
  wp_run<KSD>(K4, pi, sA, lane, [&] { wp_start(p2, a.Wkv, KSD, ng2, 0, lane); });
  bias_store<4>(K4, ng4, a.bkv, a.kv_out, 2 * kWidth, lane, row0, T);
  zero(H);
  wp_run<KSD>(H, p2, sA, lane, NoNext());
  bias_store<2>(H, ng2, a.bkv, a.kv_out, 2 * kWidth, lane, row0, T);
}

}  // namespace

hipError_t launch_layer(const LayerArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.qkv_bias_next != nullptr)
    layer_kernel<true><<<(a.T + RB - 1) / RB, 512, 0, s>>>(a);
  else
    layer_kernel<false><<<(a.T + RB - 1) / RB, 512, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_head_layer(const HeadArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  head_kernel<<<(a.T + RB - 1) / RB, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace jl
