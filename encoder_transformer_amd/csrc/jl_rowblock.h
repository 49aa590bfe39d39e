// Building blocks of the row-block kernels (bf16): 64 token rows per
// work-group of 512 threads (8 waves, two per SIMD), the rows resident in LDS
// and registers from one projection to the next.
//
// Weights stream from L2 straight into matrix-core fragments: at load they
// are pre-packed so that each (16 output columns x 32 k) block is the 1 KB a
// wave consumes, one coalesced buffer load; every GEMM runs on a "weight
// pipe" whose first k-steps were issued during the previous GEMM or before
// an epilogue.  Activations (LayerNorm outputs, feed-forward chunks) sit in
// LDS in fragment order.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16 with the weight fragment as the A
// operand and the activation fragment as B, so the accumulator is C^T: lane
// (r16 + 16 g) holds row r16 of the 16-row sub-tile and the 4 consecutive
// columns 4g .. 4g+3 of the 16-column sub-tile.  Row statistics then reduce
// over 4 lanes, and every epilogue access is a 16-byte (FP32) or 8-byte (bf16)
// vector.  A wave's model-width tile X[4][3] holds rows 16 i + r16 and columns
// 48 w + 16 j + 4 g + r.
#pragma once

#include "jl_device.h"

// No FMA contraction: unrolled code handles each row of a tile in its own
// instruction sequence, and a contraction the compiler applies to some of
// those sequences and not to others would make a row's rounding depend on
// its place in the tile, and so on how the batch was packed.
#pragma clang fp contract(off)

namespace jl {
namespace rowblock {
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

// Sum over the four 16-lane rows of a wave for each lane position (lanes i,
// i + 16, i + 32, i + 48) by the row-swap permutes, without an LDS round trip;
// every lane gets the same (r0 + r1) + (r2 + r3).
DI float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float p = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Row statistics of the 64 x 384 tile X: wave w holds columns 48w .. 48w+47 as
// 3 sub-tiles; lane (r16 + 16 g) holds row 16 i + r16, columns 16 j + 4 g + r.
// Two passes (mean, then the mean of squared deviations), reduced over the 4
// lane groups and then over the 8 waves through LDS: sRed[0] holds the
// partial sums, sRed[1] the partial squared deviations, so one barrier per
// pass suffices -- a later call cannot overwrite either buffer before every
// wave has passed the barrier that follows its last read.
DI void row_stats(const f32x4 (&X)[4][3], float (*sRed)[NW][RB], int lane, int wave, float (&mean)[4],
                  float (&rstd)[4]) {
  const int r16 = lane & 15, g = lane >> 4;
  float part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j) s += (X[i][j][0] + X[i][j][1]) + (X[i][j][2] + X[i][j][3]);
    part[i] = rows_sum(s);
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sRed[0][wave][16 * i + r16] = part[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * i + r16;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += sRed[0][w][row];
    mean[i] = t * (1.0f / kWidth);
  }
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
    part[i] = rows_sum(s);
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sRed[1][wave][16 * i + r16] = part[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * i + r16;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += sRed[1][w][row];
    rstd[i] = rsqrtf(t * (1.0f / kWidth) + kLnEps);
  }
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

// Pipe types by fragment columns per wave: 3 (model-width outputs: out-
// projections, v), 4 (MLP input chunks, whole-head q/k), 2 (the last MLP input
// chunk, half-head q/k, head feed-forward chunks).
constexpr int PDO = 3, PDI = 2, PD2 = 4;
using PipeO = WPipe<3, PDO>;
using PipeI = WPipe<4, PDI>;
using Pipe2 = WPipe<2, PD2>;

template <int NTA>
DI void zero_cols(f32x4 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NTA; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// The QKV projection's q/k of one whole head (wave w: head w) or of half a head
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
DI void start_qk_whole(PipeI &w, const bf16 *Wqkv, int lane, int wave) {
  int ng[4];
  ng_qk_whole(ng, wave);
  wp_start(w, Wqkv, KSD, ng, 0, lane);
}
DI void start_qk_half(Pipe2 &w, const bf16 *Wqkv, int lane, int wave) {
  int ng[2];
  ng_qk_half(ng, wave);
  wp_start(w, Wqkv, KSD, ng, 0, lane);
}
DI void start_v(PipeO &w, const bf16 *Wqkv, int lane, int wave) {
  int ng[3];
  ng_v(ng, wave);
  wp_start(w, Wqkv, KSD, ng, 0, lane);
}

// RoPE on q/k accumulators and store: NT = 4 holds a whole head (columns
// head_col .. head_col + 63, groups d 0-15, 16-31, 32-47, 48-63), NT = 2 the
// half `half` (groups d 16 half .. and d 32 + 16 half ..).  Rotation pairs
// are (d, d + 32).
template <int NT>
DI void rope_store(const f32x4 (&H)[4][4], const float *sCos, const float *sSin, bf16 *qkv_out, int head_col,
                   int half, int lane, int row0, int T) {
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
      bf16 *q = qkv_out + (size_t)row * (3 * kWidth) + head_col + d0;
      *reinterpret_cast<bf16x4 *>(q) = lo;
      *reinterpret_cast<bf16x4 *>(q + 32) = hi;
    }
  }
}

// rope_store<4> through a per-wave LDS tile (64 rows x 64 columns, 16-byte
// chunks XOR-swizzled by row so that the 16-byte reads are free of bank
// conflicts): each global store instruction then
// writes 8 whole 128-byte rows of the head instead of 16 rows x 32 bytes.
// The same values reach the same addresses; only the store pattern differs.
DI void rope_store_staged(const f32x4 (&H)[4][4], const float *sCos, const float *sSin, bf16 *qkv_out, int head_col,
                          bf16 *sStage, int lane, int row0, int T) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jp = 0; jp < 2; ++jp) {
    const int d0 = 16 * jp + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 16 * i + r16, sw = rl & 7;
      const f32x4 cs = *reinterpret_cast<const f32x4 *>(sCos + rl * 32 + d0);
      const f32x4 sn = *reinterpret_cast<const f32x4 *>(sSin + rl * 32 + d0);
      bf16x4 lo, hi;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = H[i][jp][r], x1 = H[i][jp + 2][r];
        lo[r] = (bf16)(x0 * cs[r] - x1 * sn[r]);
        hi[r] = (bf16)(x1 * cs[r] + x0 * sn[r]);
      }
      *reinterpret_cast<bf16x4 *>(sStage + rl * 64 + (((d0 >> 3) ^ sw) << 3) + (d0 & 7)) = lo;
      *reinterpret_cast<bf16x4 *>(sStage + rl * 64 + ((((d0 + 32) >> 3) ^ sw) << 3) + (d0 & 7)) = hi;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rl = 8 * k + (lane >> 3), c = lane & 7, row = row0 + rl;
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(sStage + rl * 64 + ((c ^ (rl & 7)) << 3));
    if (row < T) *reinterpret_cast<bf16x8 *>(qkv_out + (size_t)row * (3 * kWidth) + head_col + 8 * c) = v;
  }
}

// The e4m3 QKV phase computes a whole head in two rotation halves: each
// half's rotated q/k values (columns 16 hf + (0..15) and + 32) go into the
// wave's swizzled head tile as rope_store_staged lays it out, and
// head_tile_store writes the tile after the second half.
DI void rope_stage_half(const f32x4 (&H)[4][4], const float *sCos, const float *sSin, int hf, bf16 *sStage,
                        int lane) {
  const int r16 = lane & 15, g = lane >> 4, d0 = 16 * hf + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 16 * i + r16, sw = rl & 7;
    const f32x4 cs = *reinterpret_cast<const f32x4 *>(sCos + rl * 32 + d0);
    const f32x4 sn = *reinterpret_cast<const f32x4 *>(sSin + rl * 32 + d0);
    bf16x4 lo, hi;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x0 = H[i][0][r], x1 = H[i][1][r];
      lo[r] = (bf16)(x0 * cs[r] - x1 * sn[r]);
      hi[r] = (bf16)(x1 * cs[r] + x0 * sn[r]);
    }
    *reinterpret_cast<bf16x4 *>(sStage + rl * 64 + (((d0 >> 3) ^ sw) << 3) + (d0 & 7)) = lo;
    *reinterpret_cast<bf16x4 *>(sStage + rl * 64 + ((((d0 + 32) >> 3) ^ sw) << 3) + (d0 & 7)) = hi;
  }
}
DI void head_tile_store(const bf16 *sStage, bf16 *qkv_out, int head_col, int lane, int row0, int T) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rl = 8 * k + (lane >> 3), c = lane & 7, row = row0 + rl;
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(sStage + rl * 64 + ((c ^ (rl & 7)) << 3));
    if (row < T) *reinterpret_cast<bf16x8 *>(qkv_out + (size_t)row * (3 * kWidth) + head_col + 8 * c) = v;
  }
}

// v_store through a per-wave LDS tile (64 rows x 48 columns, rows 112 bytes
// apart): each global store instruction then writes 96-byte row segments
// instead of 32-byte ones.
DI void v_store_staged(const f32x4 (&V)[4][3], bf16 *qkv_out, bf16 *sStage, int lane, int wave, int row0, int T) {
  constexpr int S = 56;  // tile row stride (elements)
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      bf16x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (bf16)V[i][j][r];
      *reinterpret_cast<bf16x4 *>(sStage + (16 * i + r16) * S + 16 * j + 4 * g) = t;
    }
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const int q = 64 * k + lane, rl = q / 6, c = q - 6 * rl, row = row0 + rl;
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(sStage + rl * S + 8 * c);
    if (row < T) *reinterpret_cast<bf16x8 *>(qkv_out + (size_t)row * (3 * kWidth) + 2 * kWidth + 48 * wave + 8 * c) = v;
  }
}

// v accumulators (wave w: columns 48 w .. 48 w + 47) to bf16.
DI void v_store(const f32x4 (&V)[4][3], bf16 *qkv_out, int lane, int wave, int row0, int T) {
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 16 * i + r16;
    if (row >= T) continue;
    bf16 *v = qkv_out + (size_t)row * (3 * kWidth) + 2 * kWidth + 48 * wave + 4 * g;
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


// The QKV projection of the fragment-order LayerNorm output sA (64 x 384):
// q and k (12 heads): heads 0-7 one per wave, heads 8-11 two waves each; v:
// 48 columns per wave.  Waves 0-3 take [whole head, half head, v], waves 4-7
// [half head, v, whole head], so that one wave's epilogue overlaps its SIMD
// partner's matrix-core work.  kBias: add the projection bias and store
// (the head's in-projection); else rotate q and k (RoPE rows of this block in
// sCos / sSin) and store.  Every pipe, H and X are free on entry.
// sStage: this wave's 8 KB of free LDS, through which the encoder's whole-head
// q/k and v stores are staged (nullptr: stored straight from registers).
template <bool kBias>
DI void qkv_phase(const bf16 *Wqkv, const float *bias, bf16 *qkv_out, const float *sCos, const float *sSin,
                  const bf16 *sA, PipeO &po, PipeI &pi, Pipe2 &p2, f32x4 (&H)[4][4], f32x4 (&X)[4][3], int lane,
                  int wave, int row0, int T, bf16 *sStage = nullptr) {
  const int half_col = 512 + 64 * (wave >> 1), half = wave & 1;
  int ngw[4], ngh[2], ngv[3];
  ng_qk_whole(ngw, wave);
  ng_qk_half(ngh, wave);
  ng_v(ngv, wave);
  constexpr int QS = 3 * kWidth;
  if (wave < NW / 2) {
    start_qk_whole(pi, Wqkv, lane, wave);
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, [&] { start_qk_half(p2, Wqkv, lane, wave); });
    if constexpr (kBias) bias_store<4>(H, ngw, bias, qkv_out, QS, lane, row0, T);
    else if (sStage) rope_store_staged(H, sCos, sSin, qkv_out, 64 * wave, sStage, lane, row0, T);
    else rope_store<4>(H, sCos, sSin, qkv_out, 64 * wave, 0, lane, row0, T);
    zero_cols<2>(H);
    wp_run<KSD>(H, p2, sA, lane, [&] { start_v(po, Wqkv, lane, wave); });
    if constexpr (kBias) bias_store<2>(H, ngh, bias, qkv_out, QS, lane, row0, T);
    else rope_store<2>(H, sCos, sSin, qkv_out, half_col, half, lane, row0, T);
    zero(X);
    wp_run<KSD>(X, po, sA, lane, NoNext());
    if constexpr (kBias) bias_store<3>(X, ngv, bias, qkv_out, QS, lane, row0, T);
    else if (sStage) v_store_staged(X, qkv_out, sStage, lane, wave, row0, T);
    else v_store(X, qkv_out, lane, wave, row0, T);
  } else {
    start_qk_half(p2, Wqkv, lane, wave);
    zero_cols<2>(H);
    wp_run<KSD>(H, p2, sA, lane, [&] { start_v(po, Wqkv, lane, wave); });
    if constexpr (kBias) bias_store<2>(H, ngh, bias, qkv_out, QS, lane, row0, T);
    else rope_store<2>(H, sCos, sSin, qkv_out, half_col, half, lane, row0, T);
    zero(X);
    wp_run<KSD>(X, po, sA, lane, [&] { start_qk_whole(pi, Wqkv, lane, wave); });
    if constexpr (kBias) bias_store<3>(X, ngv, bias, qkv_out, QS, lane, row0, T);
    else if (sStage) v_store_staged(X, qkv_out, sStage, lane, wave, row0, T);
    else v_store(X, qkv_out, lane, wave, row0, T);
    zero_cols<4>(H);
    wp_run<KSD>(H, pi, sA, lane, NoNext());
    if constexpr (kBias) bias_store<4>(H, ngw, bias, qkv_out, QS, lane, row0, T);
    else if (sStage) rope_store_staged(H, sCos, sSin, qkv_out, 64 * wave, sStage, lane, row0, T);
    else rope_store<4>(H, sCos, sSin, qkv_out, 64 * wave, 0, lane, row0, T);
  }
}

// ---------------------------------------------------------------------------
// e4m3 products (JL_FP8): v_mfma_scale_f32_16x16x128_f8f6f4 with unit block
// scales, 128 k per product.  A fragment block (16 rows x 128 k) is 2 KB:
// half h (k 16 h .. 16 h + 15 of each lane's 32) is 1 KB, lane l holding row
// l % 16, k = 32 (l / 16) + 16 h + e.  Weights are packed in this order
// (blocks gn-major, then k-step), and the LayerNorm output tile in LDS uses
// it too (row group i, k-step s at block 3 i + s), so every load is one
// contiguous 1 KB wave access.
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int KS8 = kWidth / 128;  // 3 k-steps of 128 over the model width

DI i32x8 cat8(i32x4 lo, i32x4 hi) { return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }
DI __amdgpu_buffer_rsrc_t codes_rsrc(const uint8_t *W) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), (short)0, 0x7fffffff, 0x00020000);
}
DI i32x8 ldw8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return cat8(__builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0)),
              __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 1024, 0)));
}
DI i32x8 lds_frag8(const uint8_t *p) {
  return cat8(*reinterpret_cast<const i32x4 *>(p), *reinterpret_cast<const i32x4 *>(p + 1024));
}

// An e4m3 weight pipe: PD of the 3 k-steps of a wave's NT fragment columns in flight.
template <int NT, int PD>
struct WPipe8 {
  const uint8_t *W;
  int vo[NT];
  i32x8 fb[PD][NT];
};

template <int NT, int PD>
DI void wp8_start(WPipe8<NT, PD> &w, const uint8_t *Wp, const int (&ng)[NT], int lane) {
  static_assert(PD <= KS8, "prefetch depth");
  w.W = Wp;
  const __amdgpu_buffer_rsrc_t rw = codes_rsrc(Wp);
#pragma unroll
  for (int j = 0; j < NT; ++j) w.vo[j] = ng[j] * (KS8 * 2048) + lane * 16;
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int j = 0; j < NT; ++j) w.fb[p][j] = ldw8(rw, w.vo[j], p * 2048);
}

// acc[i][j] += (codes(A) . codes(W)^T)^T over the 384-wide e4m3 tile sA8 for a
// started pipe (the unscaled sums of code products).  A weight fragment is
// reloaded right after the products that read it (with PD = 1 the next
// column's products then cover its latency); the activation fragments of the
// next k-step are read once every column is done.  `next()` runs once every
// load of this product is issued.
template <int NT, int PD, int NTA, class Next>
DI void wp8_run(f32x4 (&acc)[4][NTA], WPipe8<NT, PD> &w, const uint8_t *sA8, int lane, Next next) {
  static_assert(NT <= NTA, "accumulator columns");
  // the tile is read afresh by every product: kept from one product to the
  // next, all its fragments (96 registers) would stay live
  asm volatile("" ::: "memory");
  const __amdgpu_buffer_rsrc_t rw = codes_rsrc(w.W);
  const uint8_t *ap = sA8 + lane * 16;
  i32x8 fa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = lds_frag8(ap + (i * KS8) * 2048);
#pragma unroll
  for (int s = 0; s < KS8; ++s) {
    const int p = s % PD;
    if (s == KS8 - PD) next();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.fb[p][j], fa[i], acc[i][j], 0, 0, 0, 127, 0,
                                                                     127);
      if (s + PD < KS8) w.fb[p][j] = ldw8(rw, w.vo[j], (s + PD) * 2048);
    }
    if (s + 1 < KS8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds_frag8(ap + (i * KS8 + s + 1) * 2048);
    }
    // a k-step's loads stay in it: no load of a later step moves up (that
    // would keep all three steps' fragments live at once)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The e4m3 LayerNorm tile: y = gain * (X - mean) * rstd (+ shift) in FP32 as
// in write_ln, each row's largest magnitude over all 384 columns (reduced
// over the 4 lane groups and the 8 waves through sAmax, one barrier), codes
// of y * fl(448 / amax) into sA8, and the row scale fl(amax / 448) (1 for an
// all-zero row) returned per row group of this lane.
template <bool kShift>
DI void write_ln8(const f32x4 (&X)[4][3], const float *__restrict__ gain, const float *__restrict__ shift,
                  const float (&mean)[4], const float (&rstd)[4], float (*sAmax)[RB], uint8_t *sA8,
                  float (&srow)[4], int lane, int wave) {
  const int r16 = lane & 15, g = lane >> 4;
  f32x4 y[4][3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int col = 48 * wave + 16 * j + 4 * g;
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(gain + col);
    f32x4 sh = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kShift) sh = *reinterpret_cast<const f32x4 *>(shift + col);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[i][j][r] = (X[i][j][r] - mean[i]) * rstd[i] * gm[r];
        if constexpr (kShift) y[i][j][r] = y[i][j][r] + sh[r];
      }
  }
  float am[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) a = fmaxf(a, fabsf(y[i][j][r]));
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    am[i] = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sAmax[wave][16 * i + r16] = am[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) a = fmaxf(a, sAmax[w][16 * i + r16]);
    const float rc = a > 0.f ? 448.0f / a : 1.0f;
    srow[i] = a > 0.f ? a / 448.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      // columns k .. k+3 of row 16 i + r16: k-step k / 128, lane group
      // (k % 128) / 32, half (k % 32) / 16, byte k % 16
      const int k = 48 * wave + 16 * j + 4 * g, kk = k & 127;
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[i][j][0] * rc, y[i][j][1] * rc, 0, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(y[i][j][2] * rc, y[i][j][3] * rc, c, true);
      *reinterpret_cast<int *>(sA8 + ((i * KS8 + (k >> 7)) * 2 + ((kk >> 4) & 1)) * 1024 +
                               (r16 + 16 * (kk >> 5)) * 16 + (kk & 15)) = c;
    }
  }
}

// H[i][j] *= srow[i] * scale(column): the e4m3 products' scales, column scales
// of fragment group ng[j] (16 columns) from `cs`.
template <int NT, int NTA>
DI void scale8(f32x4 (&H)[4][NTA], const int (&ng)[NT], const float *cs, const float (&srow)[4], int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const f32x4 c = *reinterpret_cast<const f32x4 *>(cs + 16 * ng[j] + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) H[i][j][r] = H[i][j][r] * (srow[i] * c[r]);
  }
}

// An empty instruction that reads accumulators: the products that produce
// them are complete here, not sunk into the epilogue's per-row branches
// (which would keep every fragment they read live until then).  Emits no
// code.
template <int NT, int NTA>
DI void pin_acc(const f32x4 (&H)[4][NTA]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) asm volatile("" ::"v"(H[i][j]));
}

using PipeO8 = WPipe8<3, 1>;
using Pipe28 = WPipe8<2, 1>;

// The QKV projection with e4m3 operands (the codes of the LayerNorm tile sA8,
// row scales srow), in qkv_phase's order, each q/k head taken as its two
// rotation halves (column groups d, d + 32), so that one product keeps 32
// accumulators live; then RoPE on q and k and the stores.
DI void qkv_phase8(const uint8_t *Wqkv8, const float *sqkv, bf16 *qkv_out, const float *sCos, const float *sSin,
                   const uint8_t *sA8, const float (&srow)[4], PipeO8 &po, Pipe28 &pa, Pipe28 &pb, f32x4 (&H)[4][4],
                   f32x4 (&X)[4][3], int lane, int wave, int row0, int T, bf16 *sStage) {
  const int half_col = 512 + 64 * (wave >> 1), half = wave & 1;
  const int ngw0[2] = {4 * wave, 4 * wave + 2}, ngw1[2] = {4 * wave + 1, 4 * wave + 3};
  int ngh[2], ngv[3];
  ng_qk_half(ngh, wave);
  ng_v(ngv, wave);
  // the next product's pipe starts once this one's products are issued, its
  // loads in flight during the epilogue
  // whole: a rotation half of the wave's own head, staged (the second half
  // then writes the head's rows); else half of a shared head, stored directly
  auto qk_half = [&](Pipe28 &p, const int (&ng)[2], int col, int hf, bool whole, auto nxt) {
    zero_cols<2>(H);
    wp8_run(H, p, sA8, lane, NoNext());
    scale8<2>(H, ng, sqkv, srow, lane);
    pin_acc<2>(H);
    nxt();
    if (whole) {
      rope_stage_half(H, sCos, sSin, hf, sStage, lane);
      if (hf == 1) head_tile_store(sStage, qkv_out, col, lane, row0, T);
    } else {
      rope_store<2>(H, sCos, sSin, qkv_out, col, hf, lane, row0, T);
    }
  };
  auto v_part = [&](auto nxt) {
    zero(X);
    wp8_run(X, po, sA8, lane, NoNext());
    scale8<3>(X, ngv, sqkv, srow, lane);
    pin_acc<3>(X);
    nxt();
    v_store_staged(X, qkv_out, sStage, lane, wave, row0, T);
  };
  if (wave < NW / 2) {
    wp8_start(pa, Wqkv8, ngw0, lane);
    qk_half(pa, ngw0, 64 * wave, 0, true, [&] { wp8_start(pb, Wqkv8, ngw1, lane); });
    qk_half(pb, ngw1, 64 * wave, 1, true, [&] { wp8_start(pa, Wqkv8, ngh, lane); });
    qk_half(pa, ngh, half_col, half, false, [&] { wp8_start(po, Wqkv8, ngv, lane); });
    v_part(NoNext());
  } else {
    wp8_start(pa, Wqkv8, ngh, lane);
    qk_half(pa, ngh, half_col, half, false, [&] { wp8_start(po, Wqkv8, ngv, lane); });
    v_part([&] { wp8_start(pb, Wqkv8, ngw0, lane); });
    qk_half(pb, ngw0, 64 * wave, 0, true, [&] { wp8_start(pa, Wqkv8, ngw1, lane); });
    qk_half(pa, ngw1, 64 * wave, 1, true, NoNext());
  }
}

// Stage the RoPE table rows of this block's positions (one per row, from
// pos_of(r)) in LDS: 64 rows x 32 angles of each table.
template <class PosOf>
DI void stage_rope(float *sCos, float *sSin, const float *cos_t, const float *sin_t, int tid, PosOf pos_of) {
  for (int c = tid; c < RB * 8; c += 512) {
    const int r = c >> 3, q = (c & 7) * 4;
    const int p = pos_of(r);
    *reinterpret_cast<f32x4 *>(&sCos[r * 32 + q]) = *reinterpret_cast<const f32x4 *>(cos_t + p * 32 + q);
    *reinterpret_cast<f32x4 *>(&sSin[r * 32 + q]) = *reinterpret_cast<const f32x4 *>(sin_t + p * 32 + q);
  }
}

}  // namespace rowblock
}  // namespace jl
